"""Benchmark of the NF4-dequant-fused input-gradient GEMM on one MI355X.

One "step" is the input-gradient work of one training step of a 7B-class
decoder with NF4-frozen base weights: 28 layers x 7 projections (q, k, v, o,
gate, up, down) at M = 8192 tokens, issued in backward order (layer 27 -> 0;
down, up, gate, o, v, k, q), 196 calls of nf4_grad_a.  Inputs are synthetic
and resident in HBM before timing: weights ~ N(0, 0.02) quantised on the
device with nf4_pack, grad_out ~ N(0, 1e-2).

Printed on stdout: ONE JSON line.  `value` is whole-step throughput in
TFLOP/s (2*M*N*K summed over the 196 calls, divided by the measured step
time).  `roofline` covers the dominant kernel -- the grad_A kernel with the
most time in the step -- from HIP events recorded around every call inside
the timed steps: achieved = its FLOPs / its summed launch durations.
`traffic` is the HBM bytes per launch from the committed counter summary in
profiles/, reported only when that summary was taken on the current kernel
source.  `cpu_baseline` is the fp64 CPU oracle timed on a bounded sample.
`per_config` holds the four smaller workloads (tiny, attention projection,
MLP pair, skinny sweep), timed with rotated input sets so they do not sit in
the 256 MB Infinity Cache; `per_config_forward` the same layers' forward
product and `per_config_rms_norm` the RMSNorm backward (algorithmic GB/s).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-configs]
       python bench.py --forward-configs | --unfused-configs | --rmsnorm-configs | --aux-configs | --grouped-skinny
                                                                                                   (side tables)
       python bench.py --one M,N,K [--steps K] [--warmup W]   (one shape, for counter collection)
       python bench.py --copy-calibration   (1 GiB device copy, for counter scaling)
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

PEAK_FP16_TFLOPS = 2500.0   # MI355X dense fp16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published

LAYERS = 28
PROJ = [("q", 3584, 3584), ("k", 512, 3584), ("v", 512, 3584), ("o", 3584, 3584),
        ("gate", 18944, 3584), ("up", 18944, 3584), ("down", 3584, 18944)]
BACKWARD_ORDER = ["down", "up", "gate", "o", "v", "k", "q"]
M_STEP = 8192


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(M, N, K):
    return 4 * M * N + K * N // 2 + K * N // 16 + 4 * M * K


def roofline_time(M, N, K):
    return max(2.0 * M * N * K / (PEAK_FP16_TFLOPS * 1e12), alg_bytes(M, N, K) / (PEAK_HBM_GBS * 1e9))


def build_full_step(torch, nb):
    """Packed weights for all 196 projections, one grad_out and one grad_A per projection type."""
    gen = torch.Generator(device="cuda")
    weights = {}
    for layer in range(LAYERS):
        for pi, (p, N, K) in enumerate(PROJ):
            gen.manual_seed(1000 * layer + pi)
            w = torch.empty((N, K), device="cuda", dtype=torch.float32)
            w.normal_(0.0, 0.02, generator=gen)
            weights[(layer, p)] = nb.pack(w)
            del w
    gen.manual_seed(7)
    gouts, outs = {}, {}
    for (p, N, K) in PROJ:
        g = torch.empty((M_STEP, N), device="cuda", dtype=torch.float32)
        g.normal_(0.0, 1e-2, generator=gen)
        gouts[p] = g
        outs[p] = torch.empty((M_STEP, K), device="cuda", dtype=torch.float32)
    torch.cuda.synchronize()
    return weights, gouts, outs


def run_step(nb, weights, gouts, outs, events=None):
    """One step: 196 calls in backward order.  With `events`, record an event pair around each call."""
    for layer in range(LAYERS - 1, -1, -1):
        for p in BACKWARD_ORDER:
            s, c = weights[(layer, p)]
            if events is not None:
                e0, e1 = events["free"].pop()
                e0.record()
                nb.grad_a(gouts[p], s, c, out=outs[p])
                e1.record()
                events["done"].append((p, e0, e1))
            else:
                nb.grad_a(gouts[p], s, c, out=outs[p])


# Projections whose grad_out becomes available together in a layer's backward pass: the MLP output
# projection first, then its two input projections, then the attention output, then q, k and v.
DEPENDENCY_GROUPS = [["down"], ["up", "gate"], ["o"], ["v", "k", "q"]]


def run_step_grouped(nb, weights, gouts, outs, groups=None):
    """The same step with grouped calls: by default each layer's 7 projections in one nf4_grad_a_grouped
    call (28 calls); with `groups`, one call per group of projections per layer."""
    for layer in range(LAYERS - 1, -1, -1):
        for grp in (groups or [BACKWARD_ORDER]):
            probs = [(gouts[p],) + tuple(weights[(layer, p)]) for p in grp]
            nb.grad_a_grouped(probs, outs=[outs[p] for p in grp])


def kernel_name_for(plan, N=None):
    """Name (as rocprofv3 reports it, without namespace and arguments) of the main kernel a plan launches."""
    if plan["kernel"] == "skinny":
        return "grad_a_skinny_kernel"
    if plan["kernel"] == "zero_fill":
        return "fill_zero_kernel"
    if plan["kernel"] == "wide":
        return "grad_a_wide_kernel<%d, 0, false>" % plan["rb"]
    if plan["kernel"] == "wide16":
        # two kernels per call: the fp16 A-fragment pass, then the wide kernel reading the fragments
        return "grad_out_frag_kernel<false>+grad_a_wide_kernel<1, 3, false>"
    if plan["kernel"] == "mid":
        return "grad_out_frag_kernel<false>+grad_a_mid_kernel<%d>" % plan["rb"]
    if plan["kernel"] == "small":
        return "grad_out_frag_kernel<false>+grad_a_small_kernel"
    if plan["kernel"] == "stream":
        return "grad_a_stream_kernel<true>" if N is not None and N % 4 == 0 else "grad_a_stream_kernel<false>"
    return "grad_a_tile_kernel<%d>" % plan["rb"]


# Device code of the dominant kernel (the fp16 fragment pass and the wide
# kernel, with their shared headers); a recorded counter summary is valid only
# for the sources it was taken on.
KERNEL_SOURCES = ("nf4_grad_a_wide.hip", "nf4_kernel_util.h", "nf4_device.h")


def source_digest():
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(here, "dequant_backward_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter summary, if it was
    taken on the current kernel source; else None."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "grad_a_full_step_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].split(": ", 1)
                vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_digest") != source_digest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def numpy_blas():
    """The BLAS numpy was built against (name and version), or None."""
    try:
        import numpy as np
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:
        return None


def device_clock_mhz(device=0):
    """Peak shader clock the HIP runtime reports (hipDeviceAttributeClockRate, kHz) for the device, read
    through the runtime copy this process already loaded (PyTorch's); None if it cannot be read."""
    import ctypes
    try:
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            return None
        hip = ctypes.CDLL(path)
        v = ctypes.c_int(0)
        hip_device_attribute_clock_rate = 5  # position of hipDeviceAttributeClockRate in hipDeviceAttribute_t
        if hip.hipDeviceGetAttribute(ctypes.byref(v), hip_device_attribute_clock_rate, device) != 0:
            return None
        return v.value / 1000.0
    except OSError:
        return None


def copy_calibration(torch):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = 256 << 20  # floats: 1 GiB
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "copies": 3}), flush=True)


def copy_bandwidth(torch, trials=5):
    """Measured device-copy bandwidth (1 GiB read + 1 GiB written per copy), for information only."""
    n = 256 << 20
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(trials):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 8.0 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return round(best, 1)


def time_config(torch, nb, M, N, K, seed, g_std, rotate_bytes=512 << 20, target_s=0.02, trials=5, op="grad_a",
                splits=1, graph=False):
    """Median per-call time of nf4_grad_a (or, op="forward", nf4_forward) over rotated input sets (each set:
    codes, scales, grad_out [M][N] or activations [M][K]): (median, min, max, input sets, per-call time of
    the same calls replayed from a HIP graph if `graph`, else None)."""
    per_set = alg_bytes(M, N, K)
    nsets = max(2, -(-rotate_bytes // per_set))
    nsets = min(nsets, 64)
    gen = torch.Generator(device="cuda")
    sets = []
    for i in range(nsets):
        gen.manual_seed(seed * 100 + i)
        w = torch.empty((N, K), device="cuda").normal_(0.0, 0.02, generator=gen)
        s, c = nb.pack(w)
        del w
        if op == "forward":
            g = torch.empty((M, K), device="cuda").normal_(0.0, g_std, generator=gen)
            o = torch.empty((M, N), device="cuda")
        else:
            g = torch.empty((M, N), device="cuda").normal_(0.0, g_std, generator=gen)
            o = torch.empty((M, K), device="cuda")
        sets.append((g, s, c, o))
    if op == "forward":
        call = nb.forward
    elif op == "unfused":
        def call(g, s, c, out):
            return nb.grad_a_forced(g, s, c, "unfused", rb=1, splits=splits, out=out)
    else:
        call = nb.grad_a
    torch.cuda.synchronize()
    for i in range(5):
        g, s, c, o = sets[i % nsets]
        call(g, s, c, out=o)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    call(*sets[0][:3], out=sets[0][3])
    torch.cuda.synchronize()
    one = max(time.perf_counter() - t0, 1e-6)
    reps = int(min(max(target_s / one, 2 * nsets), 20000))
    res = []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            g, s, c, o = sets[r % nsets]
            call(g, s, c, out=o)
        e1.record()
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) * 1e-3 / reps)
    graph_s = graph_time(torch, call, sets) if graph else None
    del sets
    torch.cuda.empty_cache()
    res.sort()
    return res[len(res) // 2], res[0], res[-1], nsets, graph_s


def graph_time(torch, call, sets, replays=20):
    """Per-call device time with the host's launch cost taken out: up to 32 calls over the rotated input
    sets captured in one HIP graph (on a stream whose workspace an eager call has sized first), replayed;
    median over `replays` replays of the elapsed time between events around a replay, per call."""
    st = torch.cuda.Stream()
    ncap = min(len(sets), 32) if len(sets) >= 8 else 4 * len(sets)
    with torch.cuda.stream(st):
        for r in range(len(sets)):
            g, s, c, o = sets[r]
            call(g, s, c, out=o)
    st.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=st):
        for r in range(ncap):
            g, s, c, o = sets[r % len(sets)]
            call(g, s, c, out=o)
    res = []
    with torch.cuda.stream(st):
        graph.replay()
        for _ in range(replays):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(st)
            graph.replay()
            e1.record(st)
            e1.synchronize()
            res.append(e0.elapsed_time(e1) * 1e-3 / ncap)
    st.synchronize()
    del graph
    res.sort()
    return res[len(res) // 2]


def unfused_splits(M, N, K):
    """N-chunk count for the unfused comparison path: the fused plan's for the 512 x 128 and 256 x 128 tile
    plans; otherwise (skinny M, small tiles) enough chunks to give every CU a 512 x 128 tile (the path has
    no skinny or small-tile kernel)."""
    tiles = -(-M // 512) * -(-K // 128)
    return max(1, min(N // 64, 256 // tiles)) if tiles < 256 else 1


def per_config_unfused(torch, nb):
    """Fused (the default plan) against the unfused comparison path -- the weights dequantised to fp16 by a
    separate pass, then the same GEMM copying them instead of decoding (bitwise the same result) -- on the
    configuration shapes and the full-step layer shapes."""
    import synth
    shapes = (synth.CONFIGS["attn_proj"] + synth.CONFIGS["mlp_pair"] + synth.SKINNY_SHAPES +
              [synth.Shape(f"full_step_{p}", M_STEP, N, K) for (p, N, K) in PROJ if p in ("q", "k", "gate", "down")])
    out = {}
    for i, shp in enumerate(shapes):
        gstd = 1.0 if shp.M <= 16 else 1e-2
        fused, _, _, _, _ = time_config(torch, nb, shp.M, shp.N, shp.K, seed=i, g_std=gstd)
        plan = nb.grad_a_plan(shp.M, shp.N, shp.K)
        fused_kernels = ("wide", "wide16", "mid")  # unsplit small tiles: the unfused path needs its own split
        sp = plan["splits"] if plan["kernel"] in fused_kernels else unfused_splits(shp.M, shp.N, shp.K)
        unf, _, _, nsets, _ = time_config(torch, nb, shp.M, shp.N, shp.K, seed=i, g_std=gstd, op="unfused", splits=sp)
        fl = 2.0 * shp.M * shp.N * shp.K
        out[shp.name] = {"M": shp.M, "N": shp.N, "K": shp.K, "fused_us": round(fused * 1e6, 2),
                         "unfused_us": round(unf * 1e6, 2), "unfused_over_fused": round(unf / fused, 3),
                         "fused_tflops": round(fl / fused / 1e12, 2), "unfused_tflops": round(fl / unf / 1e12, 2),
                         "fused_plan": plan["kernel"], "unfused_splits": sp, "rotated_input_sets": nsets}
        log(f"[bench] unfused {shp.name}: fused {fused * 1e6:.1f} us, unfused {unf * 1e6:.1f} us")
    return out


def per_config_table(torch, nb, op="grad_a"):
    """Per-configuration timing of nf4_grad_a, or (op="forward") of the same layers' forward product
    nf4_forward (activations [M][K] with the configuration's grad_out distribution, output [M][N];
    the full-step layer shapes are added for the forward)."""
    import synth
    out = {}
    plan = [("tiny", synth.CONFIGS["tiny"], 1.0), ("attn_proj", synth.CONFIGS["attn_proj"], 1e-2),
            ("mlp_pair", synth.CONFIGS["mlp_pair"], 1e-2), ("skinny", synth.SKINNY_SHAPES, 1.0)]
    if op == "forward":
        full = [synth.Shape(f"full_step_{p}", M_STEP, N, K) for (p, N, K) in PROJ if p in ("q", "k", "gate", "down")]
        plan.append(("full_step", full, 1e-2))
    for cname, shapes, gstd in plan:
        for i, shp in enumerate(shapes):
            med, lo, hi, nsets, graph_s = time_config(torch, nb, shp.M, shp.N, shp.K, seed=i, g_std=gstd, op=op,
                                                      graph=True)
            fl = 2.0 * shp.M * shp.N * shp.K
            by = alg_bytes(shp.M, shp.N, shp.K)
            tf = fl / med / 1e12
            gb = by / med / 1e9
            bound = "mfma" if fl / (PEAK_FP16_TFLOPS * 1e12) >= by / (PEAK_HBM_GBS * 1e9) else "hbm"
            out[shp.name] = {
                "M": shp.M, "N": shp.N, "K": shp.K, "us": round(med * 1e6, 2),
                "us_min": round(lo * 1e6, 2), "us_max": round(hi * 1e6, 2),
                "tflops": round(tf, 2), "gbs": round(gb, 1), "bound": bound,
                "frac_of_bound": round(tf / PEAK_FP16_TFLOPS if bound == "mfma" else gb / PEAK_HBM_GBS, 4),
                "frac_of_roofline_time": round(roofline_time(shp.M, shp.N, shp.K) / med, 4),
                "rotated_input_sets": nsets,
            }
            if graph_s is not None:
                # the same calls replayed from a HIP graph: device time without the host's per-call cost
                out[shp.name]["graph_us"] = round(graph_s * 1e6, 2)
                out[shp.name]["graph_tflops"] = round(fl / graph_s / 1e12, 2)
            if op == "grad_a":
                out[shp.name]["plan"] = nb.grad_a_plan(shp.M, shp.N, shp.K)
            log(f"[bench] {op} {shp.name}: {med * 1e6:.1f} us  {tf:.1f} TFLOP/s  {gb:.0f} GB/s")
    return out


def rms_norm_alg_bytes(rows, H):
    """x, dy read and dx written (fp32), gamma read and dgamma written, rms read."""
    return 12 * rows * H + 8 * H + 4 * rows


def per_config_rms_norm(torch, nb, rotate_bytes=512 << 20, target_s=0.02, trials=5):
    """Per-shape timing of nf4_rms_norm_backward over rotated input sets (x, gamma, rms, dy, dx, dgamma);
    HBM-bound, reported as algorithmic GB/s against the published HBM peak."""
    import synth
    out = {}
    for i, (rows, H) in enumerate(synth.RMS_NORM_SHAPES):
        per_set = rms_norm_alg_bytes(rows, H)
        nsets = min(64, max(2, -(-rotate_bytes // per_set)))
        gen = torch.Generator(device="cuda")
        sets = []
        for j in range(nsets):
            gen.manual_seed(1000 * i + j)
            x = torch.empty((rows, H), device="cuda").normal_(0.0, 1.0, generator=gen)
            dy = torch.empty((rows, H), device="cuda").normal_(0.0, 1.0, generator=gen)
            g = torch.empty((H,), device="cuda").uniform_(0.5, 1.5, generator=gen)
            r = torch.empty((rows,), device="cuda").uniform_(0.9, 1.1, generator=gen)
            sets.append((x, g, r, dy, torch.empty_like(x), torch.empty_like(g)))
        torch.cuda.synchronize()
        for j in range(5):
            a = sets[j % nsets]
            nb.rms_norm_backward(*a[:4], dx=a[4], dgamma=a[5])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        nb.rms_norm_backward(*sets[0][:4], dx=sets[0][4], dgamma=sets[0][5])
        torch.cuda.synchronize()
        one = max(time.perf_counter() - t0, 1e-6)
        reps = int(min(max(target_s / one, 2 * nsets), 20000))
        res = []
        for _ in range(trials):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for k in range(reps):
                a = sets[k % nsets]
                nb.rms_norm_backward(*a[:4], dx=a[4], dgamma=a[5])
            e1.record()
            torch.cuda.synchronize()
            res.append(e0.elapsed_time(e1) * 1e-3 / reps)
        del sets
        torch.cuda.empty_cache()
        res.sort()
        med = res[len(res) // 2]
        gb = rms_norm_alg_bytes(rows, H) / med / 1e9
        out[f"rms_norm_{rows}x{H}"] = {"rows": rows, "H": H, "us": round(med * 1e6, 2),
                                       "us_min": round(res[0] * 1e6, 2), "us_max": round(res[-1] * 1e6, 2),
                                       "alg_bytes": rms_norm_alg_bytes(rows, H), "gbs": round(gb, 1),
                                       "frac_of_hbm": round(gb / PEAK_HBM_GBS, 4), "rotated_input_sets": nsets}
        log(f"[bench] rms_norm {rows}x{H}: {med * 1e6:.2f} us  {gb:.0f} GB/s")
    return out


def per_config_aux(torch, nb, trials=5):
    """nf4_dequant and nf4_pack on the full step's largest weight (18944 x 3584), HBM-bound: algorithmic
    bytes (dequant reads codes and scales and writes fp32 weights; pack the reverse) per median call."""
    N, K = 18944, 3584
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    ws = [torch.empty((N, K), device="cuda").normal_(0.0, 0.02, generator=gen) for _ in range(2)]
    packed = [nb.pack(w) for w in ws]
    outs = [torch.empty((N, K), device="cuda") for _ in range(2)]
    code_bytes = N * K // 2 + N * K // 16
    res = {}
    for name, fn, by in [("dequant", lambda i: nb.dequant(*packed[i % 2], out=outs[i % 2]), code_bytes + 4 * N * K),
                         ("pack", lambda i: nb.pack(ws[i % 2], *packed[i % 2]), 4 * N * K + code_bytes)]:
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        tt = []
        for _ in range(trials):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(10):
                fn(i)
            e1.record()
            torch.cuda.synchronize()
            tt.append(e0.elapsed_time(e1) * 1e-3 / 10)
        tt.sort()
        med = tt[len(tt) // 2]
        res[name] = {"N": N, "K": K, "us": round(med * 1e6, 2), "alg_bytes": by, "gbs": round(by / med / 1e9, 1),
                     "frac_of_hbm": round(by / med / 1e9 / PEAK_HBM_GBS, 4)}
        log(f"[bench] {name} {N}x{K}: {med * 1e6:.1f} us  {by / med / 1e9:.0f} GB/s")
    del ws, packed, outs
    torch.cuda.empty_cache()
    return res


def per_config_grouped_skinny(torch, nb, layers=3, trials=5, op="grad_a"):
    """A 7B-class layer's seven projections at M in {1, 8, 16} (the skinny sweep's token counts): seven
    nf4_grad_a calls against one nf4_grad_a_grouped call (op="forward": nf4_forward against
    nf4_forward_grouped, activations [M, K]), per layer, weights rotated over `layers` layers so the Infinity
    Cache does not hold them.  Algorithmic bytes: codes, scales, the fp32 input and output."""
    shapes = [(n, k) for (_, n, k) in PROJ]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    W = [[(torch.empty((n, k // 64), device="cuda").uniform_(0.005, 0.05, generator=gen),
           torch.randint(0, 256, (n, k // 2), device="cuda", dtype=torch.uint8, generator=gen)) for (n, k) in shapes]
         for _ in range(layers)]
    res = {}
    for M in (1, 8, 16):
        fwd = op == "forward"
        G = [torch.empty((M, k if fwd else n), device="cuda").normal_(0.0, 1.0, generator=gen) for (n, k) in shapes]
        O = [torch.empty((M, n if fwd else k), device="cuda") for (n, k) in shapes]
        by = sum(alg_bytes(M, n, k) for (n, k) in shapes)

        def separate(l):
            for i in range(len(shapes)):
                if fwd:
                    nb.forward(G[i], W[l][i][0], W[l][i][1], out=O[i])
                else:
                    nb.grad_a(G[i], W[l][i][0], W[l][i][1], out=O[i])

        def grouped(l):
            probs = [(G[i], W[l][i][0], W[l][i][1]) for i in range(len(shapes))]
            if fwd:
                nb.forward_grouped(probs, outs=O)
            else:
                nb.grad_a_grouped(probs, outs=O)

        row = {"M": M, "layer_alg_bytes": by}
        for name, fn in (("separate", separate), ("grouped", grouped)):
            for l in range(layers):
                fn(l)
            torch.cuda.synchronize()
            tt = []
            for _ in range(trials):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for r in range(4):
                    for l in range(layers):
                        fn(l)
                e1.record()
                torch.cuda.synchronize()
                tt.append(e0.elapsed_time(e1) * 1e-3 / (4 * layers))
            tt.sort()
            med = tt[len(tt) // 2]
            row[name + "_us"] = round(med * 1e6, 2)
            row[name + "_gbs"] = round(by / med / 1e9, 1)
        log(f"[bench] skinny layer {op} M={M}: separate {row['separate_us']:.1f} us, grouped {row['grouped_us']:.1f} us")
        res[f"layer_m{M}"] = row
    del W
    torch.cuda.empty_cache()
    return res


def cpu_baseline_rms_norm(target_s=5.0):
    """The fp64 RMSNorm-backward oracle on the 8192 x 3584 shape, repeated until about `target_s` seconds."""
    import numpy as np
    import synth
    from oracle import rms_norm_oracle as ro
    rows, H = 8192, 3584
    t, n, reps = 0.0, 0, 0
    while reps == 0 or t < target_s:
        x, gamma, dy = synth.rms_norm_inputs(rows, H, seed=reps)
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1) + 1e-5).astype(np.float32)
        t0 = time.perf_counter()
        ro.rms_norm_backward(x, gamma, rms, dy)
        t += time.perf_counter() - t0
        n += rms_norm_alg_bytes(rows, H)
        reps += 1
    cores = len(os.sched_getaffinity(0))
    return {"value": round(n / t / 1e9, 3), "unit": "GB/s", "cores": min(cores, int(os.environ.get("OMP_NUM_THREADS",
                                                                                                    cores))),
            "kind": "oracle", "seconds": round(t, 2),
            "sample": f"{reps} x the 8192 x 3584 RMSNorm backward (numpy fp64), algorithmic bytes / oracle time"}


def cpu_baseline_configs(trials=3):
    """The fp64 oracle on each parity configuration (tiny, attention projection, MLP pair, skinny sweep),
    median of `trials` runs of dequant + matmul on the configuration's seeded inputs (generation excluded),
    next to the GPU's median per-call time from the per-config table when given."""
    import oracle
    import synth
    out = {}
    plan = [("tiny", synth.CONFIGS["tiny"], 1.0), ("attn_proj", synth.CONFIGS["attn_proj"], 1e-2),
            ("mlp_pair", synth.CONFIGS["mlp_pair"], 1e-2), ("skinny", synth.SKINNY_SHAPES, 1.0)]
    for _, shapes, gstd in plan:
        for i, shp in enumerate(shapes):
            b = synth.random_code_bytes(shp.N, shp.K, 100 + i)
            s = synth.random_scales_uniform(shp.N, shp.K, 101 + i)
            g = synth.grad_out_normal(shp.M, shp.N, 102 + i, std=gstd)
            tt = []
            for _ in range(trials):
                t0 = time.perf_counter()
                oracle.grad_a(g, s, b, shp.M, shp.N, shp.K, with_bound=False)
                tt.append(time.perf_counter() - t0)
            tt.sort()
            med = tt[len(tt) // 2]
            out[shp.name] = {"oracle_s": round(med, 4),
                             "oracle_tflops": round(2.0 * shp.M * shp.N * shp.K / med / 1e12, 6)}
    return out


def cpu_baseline(target_s=10.0, max_layers=8, op="grad_a"):
    """The fp64 oracle, as it stands, on a bounded sample of the full step: one layer's seven projections at
    3072 of the 8192 token rows each, repeated over further layers (fresh inputs) until about `target_s`
    seconds of oracle time have accumulated, at most `max_layers` layers.  op="forward" times the forward
    oracle on the same layers (activations [rows][K])."""
    import numpy as np
    import oracle
    import synth
    rows = 3072
    flops = 0.0
    t = 0.0
    layers = 0
    while layers < max_layers and (layers == 0 or t < target_s):
        for pi, (p, N, K) in enumerate(PROJ):
            seed = 100 * layers + pi
            b = synth.random_code_bytes(N, K, seed=seed)
            s = synth.random_scales_uniform(N, K, seed=seed + 10)
            if op == "forward":
                a = synth.grad_out_normal(rows, K, seed=seed + 20, std=1e-2)
                t0 = time.perf_counter()
                oracle.forward(a, s, b, rows, N, K, with_bound=False)
            else:
                g = synth.grad_out_normal(rows, N, seed=seed + 20, std=1e-2)
                t0 = time.perf_counter()
                oracle.grad_a(g, s, b, rows, N, K, with_bound=False)
            t += time.perf_counter() - t0
            flops += 2.0 * rows * N * K
        layers += 1
    try:
        cores = len(os.sched_getaffinity(0))
    except Exception:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": round(flops / t / 1e12, 6), "unit": "TFLOP/s", "cores": min(cores, threads),
            "kind": "oracle", "seconds": round(t, 2), "cpu_model": host_cpu_model(), "blas": numpy_blas(),
            "sample": f"{op}: {layers} layer(s) x the full step's 7 projections (q,k,v,o,gate,up,down) at {rows} "
                      f"of the 8192 token rows each: numpy fp64 dequant + matmul, {flops / 1e9:.1f} GFLOP"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table")
    ap.add_argument("--unfused-configs", action="store_true",
                    help="only the fused-against-unfused comparison table (one JSON line)")
    ap.add_argument("--forward-configs", action="store_true",
                    help="only the forward product's per-config table and its CPU oracle baseline (one JSON line)")
    ap.add_argument("--aux-configs", action="store_true",
                    help="only nf4_dequant and nf4_pack throughput on the full step's largest weight (one JSON line)")
    ap.add_argument("--grouped-skinny", action="store_true",
                    help="only the M <= 16 layer tables, separate against grouped, backward and forward (one JSON line)")
    ap.add_argument("--rmsnorm-configs", action="store_true",
                    help="only the RMSNorm backward's per-shape table and its CPU oracle baseline (one JSON line)")
    ap.add_argument("--one", type=str, default=None, metavar="M,N,K",
                    help="only run nf4_grad_a on one shape (packed N(0, 0.02) weights, grad_out N(0, 1e-2)) "
                         "--steps times after --warmup calls, for counter collection; prints one JSON line")
    ap.add_argument("--forced", type=str, default=None, metavar="KERNEL,RB,SPLITS",
                    help="with --one: run nf4_grad_a_forced with this plan (kernel name as in the binding)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the NF4 input-gradient GEMM "
              "needs no collective and is benchmarked on a single MI355X.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    import dequant_backward_gemm_amd as nb

    if args.one:
        M, N, K = (int(v) for v in args.one.split(","))
        gen = torch.Generator(device="cuda")
        gen.manual_seed(0)
        w = torch.empty((N, K), device="cuda").normal_(0.0, 0.02, generator=gen)
        s, c = nb.pack(w)
        del w
        g = torch.empty((M, N), device="cuda").normal_(0.0, 1e-2, generator=gen)
        o = torch.empty((M, K), device="cuda")
        if args.forced:
            fk, frb, fsp = args.forced.split(",")

            def call():
                nb.grad_a_forced(g, s, c, fk, rb=int(frb), splits=int(fsp), out=o)
            plan = {"forced": args.forced}
        else:
            def call():
                nb.grad_a(g, s, c, out=o)
            plan = nb.grad_a_plan(M, N, K)
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            call()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / max(args.steps, 1)
        print(json.dumps({"shape": [M, N, K], "plan": plan, "us_per_call": round(us, 2),
                          "tflops": round(2.0 * M * N * K / (us * 1e-6) / 1e12, 2)}), flush=True)
        return
    if args.unfused_configs:
        print(json.dumps({"per_config_unfused": per_config_unfused(torch, nb)}), flush=True)
        return
    if args.aux_configs:
        print(json.dumps({"per_config_aux": per_config_aux(torch, nb)}), flush=True)
        return
    if args.grouped_skinny:
        print(json.dumps({"grouped_skinny_layer": per_config_grouped_skinny(torch, nb),
                          "grouped_skinny_layer_forward": per_config_grouped_skinny(torch, nb, op="forward")}),
              flush=True)
        return
    if args.rmsnorm_configs:
        rec = {"per_config_rms_norm": per_config_rms_norm(torch, nb),
               "cpu_baseline_rms_norm": None if args.no_cpu else cpu_baseline_rms_norm()}
        print(json.dumps(rec), flush=True)
        return
    if args.forward_configs:
        rec = {"per_config_forward": per_config_table(torch, nb, op="forward"),
               "cpu_baseline_forward": None if args.no_cpu else cpu_baseline(target_s=5.0, op="forward")}
        print(json.dumps(rec), flush=True)
        return

    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    t_setup = time.perf_counter()
    weights, gouts, outs = build_full_step(torch, nb)
    log(f"[bench] full-step inputs ready in {time.perf_counter() - t_setup:.1f} s")

    step_flops = sum(2.0 * M_STEP * N * K for (_, N, K) in PROJ) * LAYERS
    step_roof = sum(roofline_time(M_STEP, N, K) for (_, N, K) in PROJ) * LAYERS

    for _ in range(args.warmup):
        run_step(nb, weights, gouts, outs)
    torch.cuda.synchronize()

    calls = LAYERS * len(PROJ)
    events = {"free": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                       for _ in range(calls * args.steps)], "done": []}
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run_step(nb, weights, gouts, outs, events)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] step {ms_per_step:.2f} ms ({value:.1f} TFLOP/s), wall {wall:.2f} s for {args.steps} steps")

    # Per-launch durations grouped by the kernel each call's plan launches; the dominant kernel is
    # the one with the most total time.
    shapes = {p: (N, K) for (p, N, K) in PROJ}
    by_kernel = {}
    for p, a, b in events["done"]:
        N, K = shapes[p]
        name = kernel_name_for(nb.grad_a_plan(M_STEP, N, K), N)
        d = by_kernel.setdefault(name, [0.0, 0.0, 0, 0.0])
        d[0] += a.elapsed_time(b) * 1e-3
        d[1] += 2.0 * M_STEP * N * K
        d[2] += 1
        d[3] += alg_bytes(M_STEP, N, K)
    dom = max(by_kernel, key=lambda k: by_kernel[k][0])
    dsec, dflop, dn, dbytes = by_kernel[dom]
    achieved = dflop / dsec / 1e12
    traffic = recorded_traffic()
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP16_TFLOPS, 4), "traffic": traffic,
            "kernel": dom, "launches": dn, "avg_launch_us": round(dsec / dn * 1e6, 1),
            "flop_per_launch": round(dflop / dn), "alg_bytes_per_launch": round(dbytes / dn),
            "share_of_step_time": round(dsec / (ms_total * 1e-3), 4),
            "kernel_source_digest": source_digest()}

    # the same step with grouped calls: each layer's projections in one call, and in the groups a
    # backward pass makes available together
    def time_grouped(groups):
        for _ in range(max(1, args.warmup)):
            run_step_grouped(nb, weights, gouts, outs, groups)
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            run_step_grouped(nb, weights, gouts, outs, groups)
        g1.record()
        torch.cuda.synchronize()
        return g0.elapsed_time(g1) / args.steps
    ms_grouped = time_grouped(None)
    ms_dep = time_grouped(DEPENDENCY_GROUPS)
    log(f"[bench] dependency-grouped step {ms_dep:.2f} ms ({step_flops / (ms_dep * 1e-3) / 1e12:.1f} TFLOP/s)")
    grouped = {"ms_per_step": round(ms_grouped, 3), "tflops": round(step_flops / (ms_grouped * 1e-3) / 1e12, 2),
               "dependency_grouped": {"groups": DEPENDENCY_GROUPS, "calls_per_step": LAYERS * len(DEPENDENCY_GROUPS),
                                      "ms_per_step": round(ms_dep, 3),
                                      "tflops": round(step_flops / (ms_dep * 1e-3) / 1e12, 2)},
               "calls_per_step": LAYERS, "frac_of_peak": round(step_flops / (ms_grouped * 1e-3) / 1e12 /
                                                               PEAK_FP16_TFLOPS, 4)}
    log(f"[bench] grouped step {ms_grouped:.2f} ms ({grouped['tflops']:.1f} TFLOP/s)")

    copy_gbs = copy_bandwidth(torch)
    per_config = None if args.no_configs else per_config_table(torch, nb)
    per_config_fwd = None if args.no_configs else per_config_table(torch, nb, op="forward")
    per_config_rms = None if args.no_configs else per_config_rms_norm(torch, nb)
    per_config_aux_ = None if args.no_configs else per_config_aux(torch, nb)
    grouped_skinny = None if args.no_configs else per_config_grouped_skinny(torch, nb)
    grouped_skinny_fwd = None if args.no_configs else per_config_grouped_skinny(torch, nb, op="forward")
    cpu = None if args.no_cpu else cpu_baseline()
    if cpu is not None:
        cpu["per_config"] = cpu_baseline_configs()
        if per_config is not None:
            for name, row in cpu["per_config"].items():
                if name in per_config:
                    row["gpu_speedup"] = round(row["oracle_s"] / (per_config[name]["us"] * 1e-6), 1)

    rec = {
        "metric": "NF4 grad_A GEMM TFLOP/s (2MNK/t) + % of MFMA or HBM roofline, per config",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "full_step: 28 layers x 7 NF4 projections (q,o 3584x3584; k,v 3584->512; gate,up "
                        "3584->18944; down 18944->3584), M=8192 tokens, NF4 block 64, fp32 grad_out/grad_A",
            "calls_per_step": LAYERS * len(PROJ),
            "step_gflop": round(step_flops / 1e9, 1),
            "step_roofline_ms": round(step_roof * 1e3, 3),
            "frac_of_roofline_time": round(step_roof * 1e3 / ms_per_step, 4),
            "device": props.name,
            "cus": props.multi_processor_count,
            "peak_clock_mhz": device_clock_mhz(),
            "copy_gbs_measured": copy_gbs,
        },
        "roofline": roof,
        "grouped_step": grouped,
        "cpu_baseline": cpu,
        "per_config": per_config,
        "per_config_forward": per_config_fwd,
        "per_config_rms_norm": per_config_rms,
        "per_config_aux": per_config_aux_,
        "grouped_skinny_layer": grouped_skinny,
        "grouped_skinny_layer_forward": grouped_skinny_fwd,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
