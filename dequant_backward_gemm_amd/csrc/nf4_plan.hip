// Launch planning and dispatch of nf4_grad_a (host code): which kernel, tile
// and split of N a shape gets, the split-N workspace and the fixed-order
// reduction of the partials.
#include <algorithm>
#include <mutex>
#include <vector>

#include "nf4_launch.h"

namespace nf4 {

// Split-N workspace: one buffer per (device, stream), grown on demand with a
// stream-ordered allocation and kept for later calls on that stream.  Calls
// on one stream run in order, so they can share it; calls on different
// streams get different buffers.  (A stream-ordered allocate/free pair per
// call cost more host time than a skinny call's kernels take.)  Each buffer
// starts with kWsCounters arrival counters, zeroed once when the buffer is
// allocated; a kernel that uses them leaves them at zero again.
namespace {
struct Workspace {
  int device;
  hipStream_t stream;
  void* ptr;
  size_t bytes;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;
}  // namespace

hipError_t stream_workspace(hipStream_t stream, size_t bytes, void** out, uint32_t** counters) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  constexpr size_t kHeader = (size_t)kWsCounters * sizeof(uint32_t);
  const size_t want = (kHeader + bytes + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);  // whole MiB
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  Workspace* w = nullptr;
  for (auto& x : g_ws)
    if (x.device == dev && x.stream == stream) w = &x;
  auto hand_out = [&]() {
    *out = static_cast<char*>(w->ptr) + kHeader;
    if (counters != nullptr) *counters = static_cast<uint32_t*>(w->ptr);
  };
  if (w != nullptr && w->bytes >= kHeader + bytes) {
    hand_out();
    return hipSuccess;
  }
  // Growing allocates (and frees the old buffer) in stream order, which must
  // not happen inside a HIP graph capture: a captured graph would own the new
  // buffer and keep a pointer to the freed one.
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return e;
  if (cap != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
  if (w == nullptr) {
    g_ws.push_back(Workspace{dev, stream, nullptr, 0});
    w = &g_ws.back();
  }
  if (w->ptr != nullptr) {
    // the stream's earlier work still uses it: released in stream order
    e = hipFreeAsync(w->ptr, stream);
    w->ptr = nullptr;
    w->bytes = 0;
    if (e != hipSuccess) return e;
  }
  e = hipMallocAsync(&w->ptr, want, stream);
  if (e != hipSuccess) {
    w->ptr = nullptr;
    return e;
  }
  w->bytes = want;
  // the counters start at zero (a fill kernel, in stream order)
  e = launch_fill_zero(1, static_cast<float*>(w->ptr), (int64_t)(kHeader / 16), stream);
  if (e != hipSuccess) return e;
  hand_out();
  return hipSuccess;
}

hipError_t release_workspaces() {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  hipError_t first = hipGetDevice(&cur);
  for (auto& w : g_ws) {
    if (w.ptr == nullptr) continue;
    // every stream of the device drained first: the owning stream may be gone
    hipError_t e = hipSetDevice(w.device);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipFreeAsync(w.ptr, nullptr);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess && first == hipSuccess) first = e;
  }
  g_ws.clear();
  hipError_t e = hipSetDevice(cur);
  return first != hipSuccess ? first : e;
}

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int kCUs = 256;

GradAPlan plan_grad_a(int64_t M, int64_t N, int64_t K) {
  GradAPlan p{};
  if (N == 0) {
    p.kernel = 2;
    p.splits = 1;
    p.n_chunk = 0;
    p.grid = (int)std::min<int64_t>(cdiv(M * K / 4, 256), 4096);
    return p;
  }
  const int64_t tiles_k = cdiv(K, 256);
  if (M <= 16 && stream_kernel_supported(M, N, K)) {
    // Streaming kernel: 128-column strips x N-chunks, up to two workgroups
    // per CU at a time.  The loop is bound by each CU's LDS table reads, and
    // its time follows the busiest SIMD: wave w of a workgroup takes k-steps
    // w, w + 8, ... of its chunk, waves w and w + 4 share a SIMD, and the
    // workgroups a CU is given add up.  Fitted to split sweeps on MI355X
    // (M = 1..16; N x K = 18944 x 3584, 3584 x 18944, 14336 x 4096,
    // 4096 x 14336, 4096 x 11008, 8960 x 1536, 1536 x 1536): ~0.55 us per
    // k-step of that SIMD load, ~1.5 us per workgroup per CU beyond the
    // first, ~0.2 us per further chunk (partials and their sum by the
    // strip's last workgroup).  E.g. 18944 x 3584: 9 chunks (252
    // workgroups, 17 steps per SIMD) 16.5 us, 18 chunks (504, 2 x 9) 18.2.
    const int64_t tk = cdiv(K, kStreamBK);
    auto wave_steps = [](int64_t steps, int w) { return steps > w ? (steps - w + 7) / 8 : 0; };
    double best = 1e30;
    for (int64_t s = 1; s <= 64; ++s) {
      const int64_t chunk = cdiv(cdiv(N, s), 32) * 32;
      const int64_t se = cdiv(N, chunk);
      if (se != s) continue;
      const int64_t steps = chunk / 32;  // k-steps of the largest chunk
      int64_t simd = 0;
      for (int j = 0; j < 4; ++j) simd = std::max(simd, wave_steps(steps, j) + wave_steps(steps, j + 4));
      const int64_t grid = tk * se;
      const int64_t per_cu = cdiv(grid, kCUs);
      const double t = 0.55e-6 * (double)(per_cu * simd) + 1.5e-6 * (double)(per_cu - 1) + 0.2e-6 * (double)(se - 1);
      if (t < best * 0.999) {
        best = t;
        p.kernel = 4;
        p.rb = 0;
        p.splits = (int)se;
        p.n_chunk = (int)chunk;
        p.grid = (int)grid;
      }
    }
    return p;
  }
  if (M <= 16) {
    // Each workgroup streams one 256-wide column strip over an N-chunk
    // (multiple of 128 rows).  Aim for ~4 workgroups per CU while keeping the
    // fp32 partials (M*K per chunk) small next to the code bytes streamed.
    p.kernel = 1;
    p.rb = 0;
    int64_t want = cdiv(4 * kCUs, tiles_k);
    const int64_t part_cap = std::max<int64_t>(1, (N * K / 2) / (20 * 4 * M * K));  // partials <= 5%
    int64_t splits = std::max<int64_t>(1, std::min(want, std::max<int64_t>(part_cap, cdiv(kCUs, tiles_k))));
    splits = std::min(splits, cdiv(N, 128));
    int64_t chunk = cdiv(cdiv(N, splits), 128) * 128;
    splits = cdiv(N, chunk);
    p.splits = (int)splits;
    p.n_chunk = (int)chunk;
    p.grid = (int)(tiles_k * splits);
    return p;
  }
  // Tile kernels: pick the kernel, its tile and the N split by a simple cost
  // model: wave-quantised MFMA time at a measured efficiency plus the
  // partial-sum traffic of a split.
  const double cu_rate = 4096.0 * 2.4e9;  // fp16 MFMA flop/s per CU
  double best = 1e30;
  // Splitting N pays only when the tiles alone leave CUs idle: measured with
  // the fragment-fed wide kernel, 96 tiles ran 28% faster split in two and 48
  // tiles 15%.  Problems under a GFLOP are launch-bound and never split.
  const bool tiny = 2.0 * (double)M * (double)N * (double)K < 1e9;
  auto consider = [&](int kernel, int param, int64_t BM, int64_t BK, int per_cu, double eff, double fixed) {
    const int64_t tiles = cdiv(M, BM) * cdiv(K, BK);
    const int64_t max_split = (tiny || tiles >= kCUs) ? 1 : cdiv(N, 64);
    for (int64_t s = 1; s <= std::min<int64_t>(max_split, 16); ++s) {
      const int64_t chunk = cdiv(cdiv(N, s), 64) * 64;
      const int64_t se = cdiv(N, chunk);
      if (se != s) continue;
      const int64_t units = tiles * se;
      const int64_t rounds = cdiv(units, (int64_t)kCUs * per_cu);
      const double t_unit = (double)BM * (double)BK * (double)chunk * 2.0 / (cu_rate * eff / per_cu);
      // + ~4 us per round that no MFMA work hides: a tile's pipeline fill and
      // its output stores (fit to wide-kernel sweeps at N = 512 .. 18944)
      double t = (double)rounds * (t_unit + 4e-6) + 3e-6 + fixed;
      // split partials: written once and read once by the reduce kernel (~5 TB/s), plus the
      // reduce launch and ~0.5 us per chunk (fit to split sweeps of the mid-size tiles)
      if (se > 1) t += 2.0 * (double)se * (double)M * (double)K * 4.0 / 5.0e12 + 8e-6 + 0.5e-6 * (double)se;
      if (t < best * 0.999) {
        best = t;
        p.kernel = kernel;
        p.rb = param;
        p.splits = (int)se;
        p.n_chunk = (int)chunk;
        p.grid = (int)units;
      }
    }
  };
  // measured on MI355X (fraction of the fp16 MFMA rate at M = 8192): tile
  // kernel with 128-row tiles (two workgroups per CU) ~0.24, 256-row tiles
  // ~0.19; wide kernel 512 x 128 tiles ~0.28; wide kernel fed by fp16 A
  // fragments ~0.40, plus its conversion pass (reads 4 and writes 2 bytes per
  // grad_out element, ~5.5 TB/s, and a launch)
  consider(0, 2, 256, 256, 1, 0.19, 0.0);
  consider(0, 1, 128, 256, 2, 0.24, 0.0);
  if (wide_kernel_supported(M, N, K)) {
    const double frag_pass = 6.0 * (double)M * (double)N / 5.5e12 + 2e-6;
    consider(3, 1, wide_tile_rows(), wide_tile_cols(), 1, 0.28, 0.0);
    consider(5, 1, wide_tile_rows(), wide_tile_cols(), 1, 0.40, frag_pass);
    // Mid-size tiles run two workgroups per CU, and the time follows the
    // busiest CU's count of them: pairs at 0.376 of its MFMA rate and an odd
    // one alone at 0.26 (fit to the sweep at 2048 x 1536 x 1536 and
    // 4096 x 1536 x 8960, where they beat the 512 x 128 tiles by 5-6%).
    // Unlike the other kernels they split small problems too: at
    // 600 x 1024 x 448 four chunks ran in 16.4 us against 24.5 unsplit.
    // One workgroup's fill and stores overlap the other's MFMAs, so only
    // ~1 us per pair of them is exposed: short reductions (N <= ~1024 at
    // M = 8192) run 2-12% faster here than on the 512 x 128 tiles.
    const int64_t tiles = cdiv(M, mid_tile_rows()) * cdiv(K, wide_tile_cols());
    const int64_t max_split = tiles >= 2 * kCUs ? 1 : cdiv(N, 64);
    for (int64_t s = 1; s <= std::min<int64_t>(max_split, 16); ++s) {
      const int64_t chunk = cdiv(cdiv(N, s), 64) * 64;
      const int64_t se = cdiv(N, chunk);
      if (se != s) continue;
      const int64_t units = tiles * se;
      const int64_t load = cdiv(units, (int64_t)kCUs);
      const double flop = (double)mid_tile_rows() * (double)wide_tile_cols() * (double)chunk * 2.0;
      double t = (double)(load / 2) * 2.0 * flop / (cu_rate * 0.376) + (double)(load % 2) * flop / (cu_rate * 0.26) +
                 (double)cdiv(load, 2) * 1e-6 + 3e-6 + frag_pass;
      if (se > 1) t += 2.0 * (double)se * (double)M * (double)K * 4.0 / 5.0e12 + 8e-6 + 0.5e-6 * (double)se;
      if (t < best * 0.999) {
        best = t;
        p.kernel = 9;
        p.rb = 1;
        p.splits = (int)se;
        p.n_chunk = (int)chunk;
        p.grid = (int)units;
      }
    }
    // 128 x 128 tiles, unsplit, where the plan above splits N only to fill
    // the CUs and one round of the small tiles fills them instead: short
    // reductions (N <= 1536) with 64..256 such tiles.  The split's partials
    // and reduce launch cost more there than the small tiles' lower MFMA
    // efficiency (measured: 2048 x 1536 x 1536 34.0 against 35.8 us in two
    // chunks, 1024 x 1536 x 1536 27.4 against 31.3, 1100 x 1024 x 1088 20.1
    // against 25.3; at N = 3584 or 4096 the split plans stay ahead by 2-45%).
    const int64_t small = cdiv(M, small_tile_rows()) * cdiv(K, wide_tile_cols());
    if (!tiny && p.splits > 1 && N <= 1536 && small >= 64 && small <= kCUs) {
      p.kernel = 10;
      p.rb = 1;
      p.splits = 1;
      p.n_chunk = (int)N;
      p.grid = (int)small;
    }
  }
  return p;
}

bool make_plan(int64_t M, int64_t N, int64_t K, int kernel, int rb, int splits, GradAPlan* out) {
  GradAPlan p{};
  if (N == 0) {
    *out = plan_grad_a(M, N, K);
    return true;
  }
  if (splits < 1 || splits > 4096) return false;
  const int64_t tiles_k = cdiv(K, 256);
  if (kernel == 1) {
    if (M > 16) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 128) * 128;
    p.kernel = 1;
    p.rb = 0;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(tiles_k * p.splits);
  } else if (kernel == 0) {
    if (rb != 1 && rb != 2) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 64) * 64;
    p.kernel = 0;
    p.rb = rb;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(cdiv(M, 128 * rb) * tiles_k * p.splits);
  } else if (kernel == 4) {
    if (!stream_kernel_supported(M, N, K)) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 32) * 32;
    p.kernel = 4;
    p.rb = 0;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(cdiv(K, kStreamBK) * p.splits);
  } else if (kernel == 8) {
    if (!lines_kernel_supported(M, N, K) || rb < 0 || rb > 5) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 16) * 16;
    p.kernel = 8;
    p.rb = rb;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(cdiv(K, kLinesBK) * p.splits);
  } else if (kernel == 5 || kernel == 6 || kernel == 9 || kernel == 10) {
    if (!wide_kernel_supported(M, N, K)) return false;
    if (kernel == 9 && rb != 1 && rb != 3) return false;
    if (kernel == 10 && rb != 1) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 64) * 64;
    const int64_t rows = kernel == 9 ? mid_tile_rows() : kernel == 10 ? small_tile_rows() : wide_tile_rows();
    p.kernel = kernel;
    p.rb = kernel == 9 ? rb : 1;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(cdiv(M, rows) * cdiv(K, wide_tile_cols()) * p.splits);
  } else if (kernel == 3) {
    if (!wide_kernel_supported(M, N, K)) return false;
    const int64_t chunk = cdiv(cdiv(N, splits), 64) * 64;
    p.kernel = 3;
    p.rb = 1;
    p.n_chunk = (int)chunk;
    p.splits = (int)cdiv(N, chunk);
    p.grid = (int)(cdiv(M, wide_tile_rows()) * cdiv(K, wide_tile_cols()) * p.splits);
  } else {
    return false;
  }
  *out = p;
  return true;
}

hipError_t launch_grad_a(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                         int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_grad_a_plan(plan_grad_a(M, N, K), grad_out, scales, codes, grad_a, M, N, K, stream);
}

// Workspace layout of a plan: split partials (when N is split), then the fp16
// A fragments (fragment-fed wide kernel), then the fp16 B fragments (unfused
// comparison path), each 256-byte aligned.
struct PlanWorkspace {
  size_t part, part_al, frag, frag_al, bfrag;
  size_t total() const { return part_al + frag_al + bfrag; }
};
static PlanWorkspace plan_workspace(const GradAPlan& p, int64_t M, int64_t N, int64_t K) {
  PlanWorkspace w{};
  if (p.kernel == 2) return w;
  w.part = p.splits > 1 ? (size_t)p.splits * (size_t)M * (size_t)K * sizeof(float) : 0;
  w.part_al = (w.part + 255) & ~(size_t)255;
  w.frag = (p.kernel == 5 || p.kernel == 6 || p.kernel == 9 || p.kernel == 10) ? wide_frag_bytes(M, N) : 0;
  w.frag_al = (w.frag + 255) & ~(size_t)255;
  w.bfrag = p.kernel == 6 ? unfused_bfrag_bytes(N, K) : 0;
  return w;
}

size_t grad_a_workspace_bytes(const GradAPlan& p, int64_t M, int64_t N, int64_t K) {
  return plan_workspace(p, M, N, K).total();
}

// ---- Fixed scratch of nf4_grad_a_noalloc ----------------------------------
// A static device array (each GPU the library runs on holds its own copy until
// the process ends).  Host code never passes its name to a kernel: the name is
// a host-side stand-in, so its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// used.  The first kWsCounters dwords are the streaming kernel's arrival
// counters, zeroed by a fill kernel on the first call's stream; kernels leave
// them at zero.  Every call on a GPU shares the array.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
std::mutex g_scratch_mutex;
std::vector<void*> g_scratch_ptr;  // device address of `scratch`, per device (null until set up)
}  // namespace

static hipError_t noalloc_scratch(hipStream_t stream, FixedScratch* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    // the counters start at zero (a kernel, in this stream's order)
    e = launch_fill_zero(1, static_cast<float*>(ptr), (int64_t)kWsCounters * 4 / 16, stream);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  constexpr size_t kHeader = (size_t)kWsCounters * sizeof(uint32_t);
  out->counters = static_cast<uint32_t*>(g_scratch_ptr[dev]);
  out->base = static_cast<char*>(g_scratch_ptr[dev]) + kHeader;
  out->bytes = kNoallocScratchBytes - kHeader;
  return hipSuccess;
}

size_t noalloc_scratch_capacity() { return kNoallocScratchBytes - (size_t)kWsCounters * sizeof(uint32_t); }

hipError_t launch_grad_a_noalloc(const float* grad_out, const float* scales, const uint8_t* codes, float* grad_a,
                                 int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const GradAPlan p = plan_grad_a(M, N, K);
  if (grad_a_workspace_bytes(p, M, N, K) > noalloc_scratch_capacity()) return hipErrorOutOfMemory;
  FixedScratch fs{};
  hipError_t e = noalloc_scratch(stream, &fs);
  if (e != hipSuccess) return e;
  return launch_grad_a_plan(p, grad_out, scales, codes, grad_a, M, N, K, stream, &fs);
}

hipError_t launch_grad_a_plan(const GradAPlan& p, const float* grad_out, const float* scales, const uint8_t* codes,
                              float* grad_a, int64_t M, int64_t N, int64_t K, hipStream_t stream,
                              const FixedScratch* fixed) {
  const uint32_t* c32 = reinterpret_cast<const uint32_t*>(codes);
  if (p.kernel == 2) return launch_fill_zero(p.grid, grad_a, M * K / 4, stream);
  float* dst = grad_a;
  float* ws = nullptr;
  void* frags = nullptr;
  void* bfrags = nullptr;
  uint32_t* counters = nullptr;
  // the streaming kernel sums its own split partials (per-strip arrival counters;
  // 32-bit byte offsets into the partials)
  const bool fused_reduce = (p.kernel == 4 || p.kernel == 8) && p.splits > 1 &&
                            cdiv(K, p.kernel == 8 ? kLinesBK : kStreamBK) <= kWsCounters &&
                            (uint64_t)p.splits * (uint64_t)M * (uint64_t)K * 4 < (1ull << 32);
  {
    const PlanWorkspace w = plan_workspace(p, M, N, K);
    if (w.total() > 0) {
      char* base = nullptr;
      if (fixed != nullptr) {
        if (w.total() > fixed->bytes) return hipErrorOutOfMemory;
        base = fixed->base;
        if (fused_reduce) counters = fixed->counters;
      } else {
        hipError_t e = stream_workspace(stream, w.total(), reinterpret_cast<void**>(&base),
                                        fused_reduce ? &counters : nullptr);
        if (e != hipSuccess) return e;
      }
      if (w.part) ws = reinterpret_cast<float*>(base);
      if (w.frag) frags = base + w.part_al;
      if (w.bfrag) bfrags = base + w.part_al + w.frag_al;
    }
    if (ws) dst = ws;
  }
  const int tiles_k = (int)cdiv(K, 256);
  hipError_t e = hipSuccess;
  if (p.kernel == 1) {
    e = launch_grad_a_skinny(p.grid, grad_out, scales, c32, dst, (int)M, (int)N, (int)K, p.n_chunk, tiles_k, stream);
  } else if (p.kernel == 4) {
    e = launch_grad_a_stream(p.grid, grad_out, scales, c32, dst, grad_a, counters, (int)M, (int)N, (int)K, p.n_chunk,
                             (int)cdiv(K, kStreamBK), p.splits, stream);
  } else if (p.kernel == 8) {
    e = launch_grad_a_lines(p.rb, p.grid, grad_out, scales, c32, dst, grad_a, counters, (int)M, (int)N, (int)K,
                            p.n_chunk, (int)cdiv(K, kLinesBK), p.splits, stream);
  } else if (p.kernel == 6) {
    e = launch_grad_a_unfused(p.grid, grad_out, frags, bfrags, scales, c32, dst, (int)M, (int)N, (int)K, p.n_chunk,
                              (int)cdiv(M, wide_tile_rows()), (int)cdiv(K, wide_tile_cols()), stream);
  } else if (p.kernel == 9 || p.kernel == 10) {
    const int rows = p.kernel == 9 ? mid_tile_rows() : small_tile_rows();
    e = launch_grad_a_mid_frag(p.rb, rows, p.grid, grad_out, frags, scales, c32, dst, (int)M, (int)N, (int)K,
                               p.n_chunk, (int)cdiv(M, rows), (int)cdiv(K, wide_tile_cols()), stream);
  } else if (p.kernel == 5) {
    e = launch_grad_a_wide_frag(p.grid, grad_out, frags, scales, c32, dst, (int)M, (int)N, (int)K, p.n_chunk,
                                (int)cdiv(M, wide_tile_rows()), (int)cdiv(K, wide_tile_cols()), stream);
  } else if (p.kernel == 3) {
    e = launch_grad_a_wide(p.grid, grad_out, scales, c32, dst, (int)M, (int)N, (int)K, p.n_chunk,
                           (int)cdiv(M, wide_tile_rows()), (int)cdiv(K, wide_tile_cols()), stream);
  } else {
    e = launch_grad_a_tile(p.rb, p.grid, grad_out, scales, c32, dst, (int)M, (int)N, (int)K, p.n_chunk,
                           (int)cdiv(M, 128 * p.rb), tiles_k, stream);
  }
  if (e != hipSuccess) return e;
  if (p.splits > 1 && !fused_reduce) {
    const int64_t n4 = M * K / 4;
    const int grid = (int)std::min<int64_t>(cdiv(n4, 256), 8192);
    e = launch_grad_a_reduce(grid, ws, grad_a, n4, p.splits, stream);
  }
  return e;
}

// Forward product: 512 x 128 tiles over (M, N); when they leave CUs idle the K
// reduction is split into chunks of whole 64-wide stages (fp32 partials in the
// stream's workspace, summed in chunk order by the reduce kernel).  splits <= 0
// picks the count by the same cost model as the backward tiles.
// Streaming forward (M <= 16): 256-column strips x K chunks of whole 128-wide
// steps, the chunk partials summed inside the kernel by each strip's last
// workgroup (the reduce kernel only past the counters' limits).
// K chunking of the streaming forward: `splits` forced (> 0) or chosen.
static void forward_stream_chunks(int64_t M, int64_t N, int64_t K, int splits, int64_t* se_out, int64_t* chunk_out) {
  const int64_t strips = forward_stream_strips(N);
  int64_t se = 1, chunk = K;
  if (splits > 0) {
    chunk = cdiv(cdiv(K, splits), 128) * 128;
    se = cdiv(K, chunk);
  } else {
    // Same per-SIMD load model as the backward streaming kernel: all 8 waves
    // of a workgroup walk its whole chunk (two waves per SIMD), ~0.55 us per
    // 128-k step of that load times the workgroups per CU, ~1.5 us per
    // workgroup per CU beyond the first, ~0.2 us per further chunk, plus the
    // partials (M x N fp32 per chunk) written and read once at ~5 TB/s.
    double best = 1e30;
    for (int64_t s = 1; s <= 64; ++s) {
      const int64_t ch = cdiv(cdiv(K, s), 128) * 128;
      const int64_t e = cdiv(K, ch);
      if (e != s) continue;
      const int64_t per_cu = cdiv(strips * e, kCUs);
      double t = 0.55e-6 * (double)(per_cu * 2 * (ch / 128)) + 1.5e-6 * (double)(per_cu - 1) + 0.2e-6 * (double)(e - 1);
      if (e > 1) t += 2.0 * (double)e * (double)M * (double)N * 4.0 / 5.0e12;
      if (t < best * 0.999) {
        best = t;
        se = e;
        chunk = ch;
      }
    }
  }
  *se_out = se;
  *chunk_out = chunk;
}

// the kernel sums its own chunk partials (per-strip arrival counters; 32-bit byte offsets)
static bool forward_stream_fused(int64_t M, int64_t N, int64_t se) {
  return se > 1 && forward_stream_strips(N) <= kWsCounters && (uint64_t)se * (uint64_t)M * (uint64_t)N * 4 < (1ull << 32);
}

static hipError_t launch_nf4_forward_stream(const float* a, const float* scales, const uint8_t* codes, float* c,
                                            int64_t M, int64_t N, int64_t K, int splits, hipStream_t stream) {
  const int64_t strips = forward_stream_strips(N);
  int64_t se = 1, chunk = K;
  forward_stream_chunks(M, N, K, splits, &se, &chunk);
  float* dst = c;
  uint32_t* counters = nullptr;
  const bool fused = forward_stream_fused(M, N, se);
  if (se > 1) {
    hipError_t e = stream_workspace(stream, (size_t)se * (size_t)M * (size_t)N * sizeof(float),
                                    reinterpret_cast<void**>(&dst), fused ? &counters : nullptr);
    if (e != hipSuccess) return e;
  }
  hipError_t e = launch_forward_stream((int)(strips * se), a, scales, reinterpret_cast<const uint32_t*>(codes), dst, c,
                                       counters, (int)M, (int)N, (int)K, (int)chunk, (int)strips, (int)se, stream);
  if (e != hipSuccess) return e;
  if (se > 1 && !fused) {
    const int64_t n4 = M * N / 4;
    e = launch_grad_a_reduce((int)std::min<int64_t>(cdiv(n4, 256), 8192), dst, c, n4, (int)se, stream);
  }
  return e;
}

// Tile kernel and K split of a forward product (M > 16): the same cost model
// as the backward tiles -- one eight-wave 512 x 128 workgroup per CU at ~0.40
// of its MFMA rate plus ~4 us per round; 256 x 128 workgroups two per CU
// (pairs at 0.376, a lone one at 0.26) plus ~1 us per pair; split partials
// written and read once plus the reduce launch -- and 128 x 128 tiles,
// unsplit, where that plan splits K only to fill the CUs, the reduction is
// short (K <= 1536) and 64..256 small tiles fill them.  Sweeps of the three
// kernels over 1..6 chunks on eight shapes (rotated inputs): the model's
// choice is the fastest plan or within 2% of it on seven, and on the eighth
// (600 x 1024 x 448) 14.1 against 11.8 us for the small tiles; against the
// 512 x 128 tiles alone it gains 15% at 2048 x 1536 x 1536 (32.7 against
// 38.7 us), 6% at 4096 x 8960 x 1536 and 8% at 8192 x 512 x 3584.
static void forward_tile_plan(int64_t M, int64_t N, int64_t K, int* kernel_out, int64_t* se_out, int64_t* chunk_out) {
  const double cu_rate = 4096.0 * 2.4e9;  // fp16 MFMA flop/s per CU
  double best = 1e30;
  auto split_cost = [&](int64_t e) {
    return e > 1 ? 2.0 * (double)e * (double)M * (double)N * 4.0 / 5.0e12 + 8e-6 + 0.5e-6 * (double)e : 0.0;
  };
  auto take = [&](double t, int kernel, int64_t e, int64_t ch) {
    if (t < best * 0.999) {
      best = t;
      *kernel_out = kernel;
      *se_out = e;
      *chunk_out = ch;
    }
  };
  const int64_t tiles = cdiv(M, forward_tile_rows(kForwardTile)) * cdiv(N, 128);
  for (int64_t s = 1; s <= (tiles < kCUs ? 16 : 1); ++s) {
    const int64_t ch = cdiv(cdiv(K, s), 64) * 64;
    const int64_t e = cdiv(K, ch);
    if (e != s) continue;
    const int64_t rounds = cdiv(tiles * e, kCUs);
    take((double)rounds * (512.0 * 128.0 * (double)ch * 2.0 / (cu_rate * 0.40) + 4e-6) + split_cost(e), kForwardTile,
         e, ch);
  }
  const int64_t mid = cdiv(M, forward_tile_rows(kForwardMid)) * cdiv(N, 128);
  for (int64_t s = 1; s <= (mid < 2 * kCUs ? 16 : 1); ++s) {
    const int64_t ch = cdiv(cdiv(K, s), 64) * 64;
    const int64_t e = cdiv(K, ch);
    if (e != s) continue;
    const int64_t load = cdiv(mid * e, kCUs);
    const double flop = 256.0 * 128.0 * (double)ch * 2.0;
    take((double)(load / 2) * 2.0 * flop / (cu_rate * 0.376) + (double)(load % 2) * flop / (cu_rate * 0.26) +
             (double)cdiv(load, 2) * 1e-6 + split_cost(e),
         kForwardMid, e, ch);
  }
  const int64_t small = cdiv(M, forward_tile_rows(kForwardSmall)) * cdiv(N, 128);
  if (*se_out > 1 && K <= 1536 && small >= 64 && small <= kCUs) {
    *kernel_out = kForwardSmall;
    *se_out = 1;
    *chunk_out = K;
  }
}

hipError_t launch_nf4_forward(const float* a, const float* scales, const uint8_t* codes, float* c, int64_t M,
                              int64_t N, int64_t K, int kernel, int splits, hipStream_t stream) {
  if (K == 0) return launch_fill_zero((int)std::min<int64_t>(cdiv(M * N / 4, 256), 4096), c, M * N / 4, stream);
  if (kernel == kForwardStream || (kernel == kForwardAuto && forward_stream_supported(M, N, K)))
    return launch_nf4_forward_stream(a, scales, codes, c, M, N, K, splits, stream);
  int fk = kernel == kForwardAuto ? kForwardTile : kernel;
  int64_t se = 1, chunk = K;
  if (splits > 0) {
    chunk = cdiv(cdiv(K, splits), 64) * 64;
    se = cdiv(K, chunk);
  } else {
    forward_tile_plan(M, N, K, &fk, &se, &chunk);
  }
  const int64_t tiles_m = cdiv(M, forward_tile_rows(fk)), tiles_n = cdiv(N, 128);
  const int64_t tiles = tiles_m * tiles_n;
  const size_t part = se > 1 ? (size_t)se * (size_t)M * (size_t)N * sizeof(float) : 0;
  const size_t part_al = (part + 255) & ~(size_t)255;
  char* base = nullptr;
  hipError_t e = stream_workspace(stream, part_al + forward_frag_bytes(M, K), reinterpret_cast<void**>(&base));
  if (e != hipSuccess) return e;
  float* dst = se > 1 ? reinterpret_cast<float*>(base) : c;
  e = launch_forward(fk, (int)(tiles * se), a, base + part_al, scales, reinterpret_cast<const uint32_t*>(codes), dst,
                     (int)M, (int)N, (int)K, (int)chunk, (int)tiles_m, (int)tiles_n, stream);
  if (e != hipSuccess) return e;
  if (se > 1) {
    const int64_t n4 = M * N / 4;
    e = launch_grad_a_reduce((int)std::min<int64_t>(cdiv(n4, 256), 8192), dst, c, n4, (int)se, stream);
  }
  return e;
}

// Grouped streaming launch (M <= 16): the problems nf4_grad_a would run on
// the streaming kernel with its split sum inside the kernel (N % 4 == 0, the
// counters and offsets within their limits) run as one grid, each with its
// own plan's workgroups, so each result is bitwise that of its own call; the
// others run through their own plans.  Problems are ordered by workgroup size
// (N-chunk), largest first, so the long workgroups start first.
static hipError_t launch_grad_a_grouped_stream(const float* const* grad_out, const float* const* scales,
                                               const uint8_t* const* codes, float* const* grad_a, const int64_t* N,
                                               const int64_t* K, int count, int64_t M, hipStream_t stream) {
  int idx[kStreamGroupMax];
  GradAPlan plans[kStreamGroupMax];
  int ng = 0;
  int64_t strips_split = 0;  // counters the split problems need
  for (int i = 0; i < count; ++i) {
    if (K[i] == 0) continue;
    const GradAPlan pl = plan_grad_a(M, N[i], K[i]);
    const int64_t tk = cdiv(K[i], kStreamBK);
    const bool fits = pl.kernel == 4 && (N[i] % 4) == 0 && ng < kStreamGroupMax &&
                      (pl.splits == 1 || ((uint64_t)pl.splits * (uint64_t)M * (uint64_t)K[i] * 4 < (1ull << 32) &&
                                          strips_split + tk <= kWsCounters));
    if (fits) {
      plans[ng] = pl;
      idx[ng++] = i;
      if (pl.splits > 1) strips_split += tk;
    } else {
      hipError_t e = launch_grad_a(grad_out[i], scales[i], codes[i], grad_a[i], M, N[i], K[i], stream);
      if (e != hipSuccess) return e;
    }
  }
  if (ng == 0) return hipSuccess;
  int order[kStreamGroupMax];
  for (int j = 0; j < ng; ++j) order[j] = j;
  std::stable_sort(order, order + ng, [&](int a, int b) { return plans[a].n_chunk > plans[b].n_chunk; });
  size_t off[kStreamGroupMax], total_bytes = 0;
  for (int j = 0; j < ng; ++j) {
    const GradAPlan& pl = plans[order[j]];
    off[j] = total_bytes;
    if (pl.splits > 1)
      total_bytes += ((size_t)pl.splits * (size_t)M * (size_t)K[idx[order[j]]] * sizeof(float) + 255) & ~(size_t)255;
  }
  char* base = nullptr;
  uint32_t* counters = nullptr;
  hipError_t e = stream_workspace(stream, std::max<size_t>(total_bytes, 256), reinterpret_cast<void**>(&base),
                                  &counters);
  if (e != hipSuccess) return e;
  StreamGroup g{};
  g.count = ng;
  g.M = (int)M;
  int begin = 0;
  int cbase = 0;
  for (int j = 0; j < ng; ++j) {
    const int i = idx[order[j]];
    const GradAPlan& pl = plans[order[j]];
    StreamProblem& w = g.p[j];
    w.G = grad_out[i];
    w.S = scales[i];
    w.C32 = reinterpret_cast<const uint32_t*>(codes[i]);
    w.grad_a = grad_a[i];
    w.N = (int)N[i];
    w.K = (int)K[i];
    w.n_chunk = pl.n_chunk;
    w.tiles_k = (int)cdiv(K[i], kStreamBK);
    w.splits = pl.splits;
    if (pl.splits > 1) {
      w.part = reinterpret_cast<float*>(base + off[j]);
      w.counters = counters + cbase;
      cbase += w.tiles_k;
    } else {
      w.part = grad_a[i];
      w.counters = nullptr;
    }
    w.begin = begin;
    w.padded = (int)cdiv(pl.grid, 8) * 8;
    begin += w.padded;
  }
  return launch_grad_a_stream_grouped(g, begin, stream);
}

// Grouped grad_A: problems the fragment-fed wide kernel takes (M > 16, N % 64
// == 0, operands below 2 GiB) run as one grid, longest reduction first;
// M <= 16 problems run as one grid of the streaming kernel (above); every
// other problem runs through its own nf4_grad_a plan.  Each grouped wide
// problem's grad_out goes through its own fragment pass first (the fragments
// of all of them share the stream's workspace).
hipError_t launch_grad_a_grouped(const float* const* grad_out, const float* const* scales,
                                 const uint8_t* const* codes, float* const* grad_a, const int64_t* N,
                                 const int64_t* K, int count, int64_t M, hipStream_t stream) {
  if (M <= 16) return launch_grad_a_grouped_stream(grad_out, scales, codes, grad_a, N, K, count, M, stream);
  int idx[kWideGroupMax];
  int ng = 0;
  for (int i = 0; i < count; ++i) {
    if (K[i] == 0) continue;
    if (M > 16 && ng < kWideGroupMax && wide_kernel_supported(M, N[i], K[i])) {
      idx[ng++] = i;
    } else {
      hipError_t e = launch_grad_a(grad_out[i], scales[i], codes[i], grad_a[i], M, N[i], K[i], stream);
      if (e != hipSuccess) return e;
    }
  }
  if (ng == 0) return hipSuccess;
  // longest reduction (largest N) first, ties in call order
  std::stable_sort(idx, idx + ng, [&](int a, int b) { return N[a] > N[b]; });
  size_t off[kWideGroupMax], total_bytes = 0;
  for (int j = 0; j < ng; ++j) {
    off[j] = total_bytes;
    total_bytes += (wide_frag_bytes(M, N[idx[j]]) + 255) & ~(size_t)255;
  }
  char* base = nullptr;
  hipError_t e = stream_workspace(stream, total_bytes, reinterpret_cast<void**>(&base));
  if (e != hipSuccess) return e;
  WideGroup g{};
  g.count = ng;
  g.M = (int)M;
  g.tiles_m = (int)cdiv(M, wide_tile_rows());
  int begin = 0;
  for (int j = 0; j < ng; ++j) {
    const int i = idx[j];
    e = launch_frag_pass(grad_out[i], base + off[j], (int)M, (int)N[i], /*natural=*/false, stream);
    if (e != hipSuccess) return e;
    WideProblem& w = g.p[j];
    w.frags = base + off[j];
    w.scales = scales[i];
    w.codes = reinterpret_cast<const uint32_t*>(codes[i]);
    w.out = grad_a[i];
    w.N = (int)N[i];
    w.K = (int)K[i];
    w.tiles_k = (int)cdiv(K[i], wide_tile_cols());
    w.tile_begin = begin;
    begin += g.tiles_m * w.tiles_k;
  }
  g.total = begin;
  return launch_grad_a_wide_grouped(g, stream);
}

// Grouped forward (M <= 16): every problem nf4_forward would run on the
// streaming kernel with its chunk sum inside the kernel runs in one grid, each
// with its own plan's strips and K-chunks (bitwise the result of its own
// call), largest chunk first; the others run through their own plans.
hipError_t launch_nf4_forward_grouped(const float* const* a, const float* const* scales, const uint8_t* const* codes,
                                      float* const* c, const int64_t* N, const int64_t* K, int count, int64_t M,
                                      hipStream_t stream) {
  int idx[kStreamGroupMax];
  int64_t se_of[kStreamGroupMax], chunk_of[kStreamGroupMax];
  int ng = 0;
  int64_t strips_split = 0;
  int tiled[kStreamGroupMax];
  int nt = 0;
  for (int i = 0; i < count; ++i) {
    if (N[i] == 0) continue;
    bool grouped = false;
    if (M <= 16 && K[i] > 0 && forward_stream_supported(M, N[i], K[i]) && ng < kStreamGroupMax) {
      int64_t se = 1, chunk = K[i];
      forward_stream_chunks(M, N[i], K[i], 0, &se, &chunk);
      const int64_t strips = forward_stream_strips(N[i]);
      if (se == 1 || (forward_stream_fused(M, N[i], se) && strips_split + strips <= kWsCounters)) {
        grouped = true;
        se_of[ng] = se;
        chunk_of[ng] = chunk;
        idx[ng++] = i;
        if (se > 1) strips_split += strips;
      }
    }
    if (!grouped) {
      // the problems nf4_forward runs on the tile kernels; the streaming ones
      // left out of the group (limits of the in-kernel chunk sum) and K = 0
      // run through nf4_forward's own launch
      if (K[i] > 0 && !forward_stream_supported(M, N[i], K[i]) && nt < kStreamGroupMax) {
        tiled[nt++] = i;
      } else {
        hipError_t e = launch_nf4_forward(a[i], scales[i], codes[i], c[i], M, N[i], K[i], kForwardAuto, 0, stream);
        if (e != hipSuccess) return e;
      }
    }
  }
  if (nt > 0) {
    // Tile-kernel problems, each with the plan nf4_forward gives it.  Problems
    // with the same activations (the same `a` and K, as q, k and v, or gate
    // and up, of one layer) share one conversion of `a` into fp16 fragments.
    // One workspace holds each distinct `a`'s fragments and the largest
    // problem's split partials (the problems run in stream order, so they can
    // reuse them), allocated before anything is launched.
    int fk[kStreamGroupMax], src[kStreamGroupMax];
    int64_t se[kStreamGroupMax], chunk[kStreamGroupMax];
    size_t frag_off[kStreamGroupMax], frag_total = 0, part_max = 0;
    for (int t = 0; t < nt; ++t) {
      const int i = tiled[t];
      forward_tile_plan(M, N[i], K[i], &fk[t], &se[t], &chunk[t]);
      src[t] = t;
      for (int u = 0; u < t; ++u)
        if (a[tiled[u]] == a[i] && K[tiled[u]] == K[i]) {
          src[t] = src[u];
          break;
        }
      if (src[t] == t) {
        frag_off[t] = frag_total;
        frag_total += (forward_frag_bytes(M, K[i]) + 255) & ~(size_t)255;
      }
      if (se[t] > 1) part_max = std::max(part_max, (size_t)se[t] * (size_t)M * (size_t)N[i] * sizeof(float));
    }
    const size_t part_al = (part_max + 255) & ~(size_t)255;
    char* base = nullptr;
    hipError_t e = stream_workspace(stream, part_al + frag_total, reinterpret_cast<void**>(&base));
    if (e != hipSuccess) return e;
    for (int t = 0; t < nt; ++t) {
      const int i = tiled[t];
      void* frags = base + part_al + frag_off[src[t]];
      if (src[t] == t) {
        e = launch_frag_pass(a[i], frags, (int)M, (int)K[i], /*natural=*/true, stream);
        if (e != hipSuccess) return e;
      }
      const int64_t tiles_m = cdiv(M, forward_tile_rows(fk[t])), tiles_n = cdiv(N[i], 128);
      float* dst = se[t] > 1 ? reinterpret_cast<float*>(base) : c[i];
      e = launch_forward_tiles(fk[t], (int)(tiles_m * tiles_n * se[t]), frags, scales[i],
                               reinterpret_cast<const uint32_t*>(codes[i]), dst, (int)M, (int)N[i], (int)K[i],
                               (int)chunk[t], (int)tiles_m, (int)tiles_n, stream);
      if (e != hipSuccess) return e;
      if (se[t] > 1) {
        const int64_t n4 = M * N[i] / 4;
        e = launch_grad_a_reduce((int)std::min<int64_t>(cdiv(n4, 256), 8192), dst, c[i], n4, (int)se[t], stream);
        if (e != hipSuccess) return e;
      }
    }
  }
  if (ng == 0) return hipSuccess;
  int order[kStreamGroupMax];
  for (int j = 0; j < ng; ++j) order[j] = j;
  std::stable_sort(order, order + ng, [&](int x, int y) { return chunk_of[x] > chunk_of[y]; });
  size_t off[kStreamGroupMax], total_bytes = 0;
  for (int j = 0; j < ng; ++j) {
    const int o = order[j];
    off[j] = total_bytes;
    if (se_of[o] > 1)
      total_bytes += ((size_t)se_of[o] * (size_t)M * (size_t)N[idx[o]] * sizeof(float) + 255) & ~(size_t)255;
  }
  char* base = nullptr;
  uint32_t* counters = nullptr;
  hipError_t e = stream_workspace(stream, std::max<size_t>(total_bytes, 256), reinterpret_cast<void**>(&base),
                                  &counters);
  if (e != hipSuccess) return e;
  ForwardStreamGroup g{};
  g.count = ng;
  g.M = (int)M;
  int begin = 0, cbase = 0;
  for (int j = 0; j < ng; ++j) {
    const int o = order[j], i = idx[o];
    ForwardStreamProblem& w = g.p[j];
    w.A = a[i];
    w.S = scales[i];
    w.C32 = reinterpret_cast<const uint32_t*>(codes[i]);
    w.c = c[i];
    w.N = (int)N[i];
    w.K = (int)K[i];
    w.k_chunk = (int)chunk_of[o];
    w.strips = forward_stream_strips(N[i]);
    w.splits = (int)se_of[o];
    if (w.splits > 1) {
      w.part = reinterpret_cast<float*>(base + off[j]);
      w.counters = counters + cbase;
      cbase += w.strips;
    } else {
      w.part = c[i];
      w.counters = nullptr;
    }
    w.begin = begin;
    w.padded = (int)cdiv((int64_t)w.strips * w.splits, 8) * 8;
    begin += w.padded;
  }
  return launch_forward_stream_grouped(g, begin, stream);
}

}  // namespace nf4
