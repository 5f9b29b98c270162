"""Benchmark of the quantization-cast hot path on one MI355X.

One step is one pass of every cast over its own synthetic workload, shaped
like DeepSeek-V3 MoE tensors:
    per_token      bf16 X[4096, 7168] -> E4M3 + fp32 scales (1 x 128 groups)
    swiglu         bf16 H[8192, 4096] (gate | up) + fp32 w[8192] -> E4M3 [8192, 2048]
    per_block      bf16 W[7168, 18432] -> E4M3 + one scale per 128 x 128 block
    per_channel_T  bf16 A[16384, 7168] -> E4M3 [7168, 16384] + scales per 128 tokens
    e2m1           bf16 X[16384, 7168] (0.5 * t3) -> packed E2M1 + scales (1 x 32)
Inputs are resident in HBM before timing starts; the step touches about
1.23 GB, five times the 256 MB last-level cache, so every kernel reads
inputs that the rest of the step has evicted.

value = algorithmic bytes of the whole step (inputs read once, codes and
scales written once) / time per step, in GB/s, over the K timed steps, which
carry no timing events. Per-kernel durations come from further steps, after
those and outside `value`, in which one kernel records HIP events from its own
dispatch on the launch stream (qcast_bench_time_next): step s times kernel
s mod 5, over max(K, 150) steps, so every kernel is timed on at least 30 of
its launches whatever K is (their average, median, 10th and 90th
percentile). The roofline object is for the kernel with the largest share of
the step. Each step kernel also carries copy_GBps, the library's streaming
copy moving the same byte count after a 1 GiB flush, and of_copy, its own
rate over that ceiling; runtime_copy_GBps is the HIP runtime's own
device-to-device hipMemcpyAsync of the same bytes and library_copy_marker_GBps
the library copy, both timed by events recorded around the call (the same
method for both, so the runtime copy is a ceiling independent of this
library); per_channel_T also
carries pattern_us, its own loads and transposed stores without the
arithmetic (qcast_bench_per_channel_T_traffic), flushed_us, the cast timed
the same way (alternating with it, each after the flush), and of_pattern,
their ratio. Each step kernel also carries "flushed": 30 dispatches, each
after a 1 GiB flush on the same stream (median, p10, p90 and GB/s at the
median), the cold-cache protocol beside the in-step timing. The CPU baseline
is the oracle (single thread) on every workload in full, on this host (about
10 s); cpu_baseline_all_cores splits the same work over up to 16 cores.

"other_kernels" times, after the step and outside `value`, the small
per-token workload X[128, 512] next to the launch floor (a 16-byte copy),
and the casts that are not among the five: cast_back of the per-token codes to bf16, the
per-token cast with 1 x 32 groups and packed UE8M0 column-major scales, the
per-token E5M6 cast and its cast_back, the cast_back of E2M1 codes,
SwiGLU with the clamp and counter, SwiGLU + per-channel cast + transpose,
the SwiGLU backward cast, the per-channel cast in the input layout, the
packed formats (E2M1, E5M6) on the per-channel, per-block and SwiGLU casts,
and the per-token cast with 1 x 32 groups and fp32 column-major scales.

    python bench.py [--gpus 1] [--steps 200] [--warmup 10]
"""
import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
MIN_TIMED_LAUNCHES = 30
METRIC = "achieved HBM GB/s (bytes in+out) and % of MI355X peak, per cast kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """HIP events created without the system-scope fence on record
    (hipEventDisableSystemFence). The kernels take them through
    qcast_bench_time_next, so each pair is recorded by one kernel's dispatch
    (hipExtLaunchKernel): its elapsed time is the kernel's own duration on
    the launch stream, with no marker packets between the kernels of a
    step."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = self.ct.c_void_p()
        if self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e

    def elapsed_ms(self, a, b):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, e):
        self.hip.hipEventDestroy(e)


def make_events(hev, n, steps):
    """Event pairs for the kernel launches that are timed: with at least two
    steps per kernel, step s times kernel s mod n only (each timed launch
    costs its dispatch about 1.6 us, so timing one launch per step keeps the
    step close to an untimed one); with fewer steps every launch is timed."""
    rotate = steps >= 2 * n
    return [[(hev.create(), hev.create()) if (not rotate or i == s % n) else None
             for i in range(n)] for s in range(steps)]


def timed_runs(fns, ev):
    """Run the closures `fns` in order once per row of `ev`; a kernel with an
    event pair records it from its own dispatch."""
    import precision_quantization_amd as pq
    for row in ev:
        for pair, fn in zip(row, fns):
            if pair is not None:
                pq.qcast_bench_time_next(*pair)
            fn()


def collect(ev, hev):
    """Per-closure sorted durations in ms of the timed launches (after a
    synchronize); frees the events."""
    import torch
    torch.cuda.synchronize()
    n = len(ev[0])
    out = [sorted(hev.elapsed_ms(*row[i]) for row in ev if row[i] is not None)
           for i in range(n)]
    for row in ev:
        for pair in row:
            if pair is not None:
                hev.destroy(pair[0])
                hev.destroy(pair[1])
    return out


def spread_us(ms):
    """Median, 10th and 90th percentile (nearest rank) of sorted durations in
    ms, as microseconds."""
    def at(q):
        return round(ms[min(len(ms) - 1, max(0, math.ceil(q * len(ms)) - 1))] * 1e3, 2)
    return {"median_us": at(0.5), "p10_us": at(0.1), "p90_us": at(0.9)}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def make_workloads():
    from precision_quantization_amd import workloads as W
    return [
        ("per_token", W.per_token_hidden()),
        ("swiglu", W.swiglu_input()),
        ("per_block", W.weight_block()),
        ("per_channel_T", W.activation_channel()),
        ("e2m1", W.student_t()),
    ]


def kernel_calls(wls, dev):
    """Per kernel: a closure launching it on the current stream into
    preallocated outputs."""
    import torch
    import precision_quantization_amd as pq
    calls = []
    for name, wl in wls:
        x = wl.x.to(dev)
        rows, cols = wl.x.shape
        if name == "per_token":
            out = torch.empty(rows, cols, dtype=torch.float8_e4m3fn, device=dev)
            sf = torch.empty(rows, cols // 128, dtype=torch.float32, device=dev)
            fn = lambda x=x, out=out, sf=sf: pq.qcast_per_token(x, "e4m3", 128, out=out, out_sf=sf)
        elif name == "swiglu":
            w = wl.w.to(dev)
            out = torch.empty(rows, cols // 2, dtype=torch.float8_e4m3fn, device=dev)
            sf = torch.empty(rows, cols // 2 // 128, dtype=torch.float32, device=dev)
            fn = lambda x=x, w=w, out=out, sf=sf: pq.qcast_swiglu_per_token(
                x, w, "e4m3", 128, out=out, out_sf=sf)
        elif name == "per_block":
            out = torch.empty(rows, cols, dtype=torch.float8_e4m3fn, device=dev)
            sf = torch.empty(rows // 128, cols // 128, dtype=torch.float32, device=dev)
            fn = lambda x=x, out=out, sf=sf: pq.qcast_per_block(x, "e4m3", 128, out=out, out_sf=sf)
        elif name == "per_channel_T":
            out = torch.empty(cols, rows, dtype=torch.float8_e4m3fn, device=dev)
            sf = torch.empty(cols, rows // 128, dtype=torch.float32, device=dev)
            fn = lambda x=x, out=out, sf=sf: pq.qcast_per_channel_T(x, "e4m3", 128, out=out,
                                                                    out_sf=sf)
        elif name == "e2m1":
            out = torch.empty(rows, cols // 2, dtype=torch.uint8, device=dev)
            sf = torch.empty(rows, cols // 32, dtype=torch.float32, device=dev)
            fn = lambda x=x, out=out, sf=sf: pq.qcast_e2m1(x, 32, out=out, out_sf=sf)
        calls.append((name, wl, fn))
    return calls


def extra_calls(wls, dev):
    """The casts beyond the five of a step (timed separately, not part of
    `value`): name, shape, algorithmic bytes, closure."""
    import torch
    import precision_quantization_amd as pq
    from precision_quantization_amd import workloads as W
    by = dict(wls)
    calls = []
    # the small per-token workload (128 x 512): far below the bandwidth
    # regime, it measures the launch floor, next to a 16-byte copy
    xs = W.per_token_small().x.to(dev)
    qs0 = torch.empty(128, 512, dtype=torch.float8_e4m3fn, device=dev)
    ss0 = torch.empty(128, 4, dtype=torch.float32, device=dev)
    calls.append(("per_token_small", [128, 512], W.per_token_small().algorithmic_bytes(),
                  lambda: pq.qcast_per_token(xs, "e4m3", 128, out=qs0, out_sf=ss0)))
    tiny_src = torch.zeros(16, dtype=torch.uint8, device=dev)
    tiny_dst = torch.empty(16, dtype=torch.uint8, device=dev)
    calls.append(("launch_floor_copy16", [16], 32,
                  lambda: pq.qcast_bench_copy(tiny_src, tiny_dst)))
    # cast_back: per-token E4M3 codes of the hidden-state workload -> bf16
    x = by["per_token"].x.to(dev)
    r, c = x.shape
    q, sf = pq.qcast_per_token(x, "e4m3", 128)
    out = torch.empty(r, c, dtype=torch.bfloat16, device=dev)
    calls.append(("cast_back", [r, c], r * c + r * (c // 128) * 4 + r * c * 2,
                  lambda q=q, sf=sf, out=out: pq.qcast_cast_back(q, sf, "e4m3", 128, out=out)))
    # per-token cast with 1 x 32 groups and packed UE8M0 column-major scales
    flags = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    shape, dt = pq.sf_layout_shape(r, c, 32, flags)
    qo = torch.empty(r, c, dtype=torch.float8_e4m3fn, device=dev)
    so = torch.empty(shape, dtype=dt, device=dev)
    calls.append(("per_token_ue8m0_g32", [r, c], 2 * r * c + r * c + shape[0] * shape[1] * 4,
                  lambda x=x, qo=qo, so=so, f=flags: pq.qcast_per_token_sf(
                      x, "e4m3", 32, sf_flags=f, out=qo, out_sf=so)))
    # E5M6 per-token cast of the hidden-state workload, and its cast_back
    q6 = torch.empty(pq.code_shape("e5m6", r, c), dtype=torch.uint8, device=dev)
    s6 = torch.empty(r, c // 128, dtype=torch.float32, device=dev)
    e5m6_bytes = 2 * r * c + r * c * 3 // 2 + r * (c // 128) * 4
    calls.append(("per_token_e5m6", [r, c], e5m6_bytes,
                  lambda x=x, q6=q6, s6=s6: pq.qcast_per_token(x, "e5m6", 128, out=q6, out_sf=s6)))
    pq.qcast_per_token(x, "e5m6", 128, out=q6, out_sf=s6)
    o6 = torch.empty(r, c, dtype=torch.bfloat16, device=dev)
    calls.append(("cast_back_e5m6", [r, c], e5m6_bytes,
                  lambda q6=q6, s6=s6, o6=o6: pq.qcast_cast_back(q6, s6, "e5m6", 128, out=o6)))
    # cast_back of the same workload's E2M1 codes (1 x 32 groups)
    q2, s2 = pq.qcast_per_token(x, "e2m1", 32)
    o2 = torch.empty(r, c, dtype=torch.bfloat16, device=dev)
    calls.append(("cast_back_e2m1", [r, c], r * c // 2 + r * (c // 32) * 4 + r * c * 2,
                  lambda q2=q2, s2=s2, o2=o2: pq.qcast_cast_back(q2, s2, "e2m1", 32, out=o2)))
    # SwiGLU with clamp and counter
    wl = by["swiglu"]
    h, w = wl.x.to(dev), wl.w.to(dev)
    r, n = wl.rows, wl.cols
    cnt = torch.zeros(1, dtype=torch.int64, device=dev)
    qs = torch.empty(r, n, dtype=torch.float8_e4m3fn, device=dev)
    ss = torch.empty(r, n // 128, dtype=torch.float32, device=dev)
    calls.append(("swiglu_clamp", [r, 2 * n], wl.algorithmic_bytes(),
                  lambda h=h, w=w, qs=qs, ss=ss, cnt=cnt: pq.qcast_swiglu_per_token_ex(
                      h, w, "e4m3", 128, swiglu_clamp=5.0, clamp_count=cnt, out=qs, out_sf=ss)))
    # SwiGLU + per-channel cast + transpose
    qt = torch.empty(n, r, dtype=torch.float8_e4m3fn, device=dev)
    st = torch.empty(n, r // 128, dtype=torch.float32, device=dev)
    calls.append(("swiglu_per_channel_T", [r, 2 * n], r * 2 * n * 2 + r * 4 + n * r + n * r // 32,
                  lambda h=h, w=w, qt=qt, st=st: pq.qcast_swiglu_per_channel_T(
                      h, w, "e4m3", 128, out=qt, out_sf=st)))
    # SwiGLU backward + per-token cast of [dgate | dup]
    hg, dvg, wg = W.swiglu_grad()
    hg, dvg, wg = hg.to(dev), dvg.to(dev), wg.to(dev)
    qb = torch.empty(r, 2 * n, dtype=torch.float8_e4m3fn, device=dev)
    sb = torch.empty(r, 2 * n // 128, dtype=torch.float32, device=dev)
    calls.append(("swiglu_backward", [r, 2 * n],
                  r * 2 * n * 2 + r * n * 2 + r * 4 + r * 2 * n + r * (2 * n // 128) * 4,
                  lambda hg=hg, dvg=dvg, wg=wg, qb=qb, sb=sb: pq.qcast_swiglu_backward_per_token(
                      hg, dvg, wg, "e4m3", 128, swiglu_clamp=6.0, out=qb, out_sf=sb)))
    # per-channel cast in the input layout
    a = by["per_channel_T"].x.to(dev)
    r, c = a.shape
    qc = torch.empty(r, c, dtype=torch.float8_e4m3fn, device=dev)
    sc = torch.empty(r // 128, c, dtype=torch.float32, device=dev)
    calls.append(("per_channel", [r, c], 2 * r * c + r * c + (r // 128) * c * 4,
                  lambda a=a, qc=qc, sc=sc: pq.qcast_per_channel(a, "e4m3", 128, out=qc,
                                                                 out_sf=sc)))

    def code_bytes(fmt, n):
        return {"e2m1": n // 2, "e5m6": n // 2 * 3}.get(fmt, n)

    def outputs(fmt, rows, cols, sf_shape):
        q = torch.empty(pq.code_shape(fmt, rows, cols), dtype=torch.uint8, device=dev)
        return q, torch.empty(sf_shape, dtype=torch.float32, device=dev)

    # the packed formats on the per-channel casts (the activation workload)
    for fmt in ("e2m1", "e5m6"):
        qT_, sT_ = outputs(fmt, c, r, (c, r // 128))
        calls.append((f"per_channel_T_{fmt}", [r, c],
                      2 * r * c + c * code_bytes(fmt, r) + c * (r // 128) * 4,
                      lambda a=a, q=qT_, s=sT_, f=fmt: pq.qcast_per_channel_T(
                          a, f, 128, out=q, out_sf=s)))
    qc2, sc2 = outputs("e2m1", r, c, (r // 128, c))
    calls.append(("per_channel_e2m1", [r, c], 2 * r * c + r * c // 2 + (r // 128) * c * 4,
                  lambda a=a, q=qc2, s=sc2: pq.qcast_per_channel(a, "e2m1", 128, out=q,
                                                                 out_sf=s)))
    # ... and on the per-block cast (the weight workload)
    wb = by["per_block"].x.to(dev)
    r, c = wb.shape
    for fmt in ("e2m1", "e5m6"):
        qb_, sb_ = outputs(fmt, r, c, (r // 128, c // 128))
        calls.append((f"per_block_{fmt}", [r, c],
                      2 * r * c + r * code_bytes(fmt, c) + (r // 128) * (c // 128) * 4,
                      lambda x=wb, q=qb_, s=sb_, f=fmt: pq.qcast_per_block(x, f, 128, out=q,
                                                                           out_sf=s)))
    # SwiGLU in the packed formats: per-token (E2M1 with 1 x 32 groups, E5M6 with
    # 1 x 128), per-channel + transpose, and the backward
    r, n = wl.rows, wl.cols
    sw_in = r * 2 * n * 2 + r * 4
    for fmt, g in (("e2m1", 32), ("e5m6", 128)):
        qs_, ss_ = outputs(fmt, r, n, (r, n // g))
        calls.append((f"swiglu_{fmt}_g{g}", [r, 2 * n],
                      sw_in + r * code_bytes(fmt, n) + r * (n // g) * 4,
                      lambda h=h, w=w, q=qs_, s=ss_, f=fmt, g=g: pq.qcast_swiglu_per_token(
                          h, w, f, g, out=q, out_sf=s)))
    qt2, st2 = outputs("e2m1", n, r, (n, r // 128))
    calls.append(("swiglu_per_channel_T_e2m1", [r, 2 * n],
                  sw_in + n * r // 2 + n * (r // 128) * 4,
                  lambda h=h, w=w, q=qt2, s=st2: pq.qcast_swiglu_per_channel_T(
                      h, w, "e2m1", 128, out=q, out_sf=s)))
    qb2, sb2 = outputs("e2m1", r, 2 * n, (r, 2 * n // 32))
    calls.append(("swiglu_backward_e2m1_g32", [r, 2 * n],
                  r * 2 * n * 2 + r * n * 2 + r * 4 + r * n + r * (2 * n // 32) * 4,
                  lambda hg=hg, dvg=dvg, wg=wg, q=qb2, s=sb2: pq.qcast_swiglu_backward_per_token(
                      hg, dvg, wg, "e2m1", 32, swiglu_clamp=6.0, out=q, out_sf=s)))
    # the scale layouts of the transposed and backward casts: packed UE8M0,
    # column-major (the activation workload, and the backward's inputs)
    pc = pq.SF_PACKED_UE8M0 | pq.SF_COL_MAJOR
    r, c = a.shape
    shape, dt = pq.sf_layout_shape(c, r, 128, pc)
    qT3 = torch.empty(c, r, dtype=torch.float8_e4m3fn, device=dev)
    sT3 = torch.empty(shape, dtype=dt, device=dev)
    calls.append(("per_channel_T_ue8m0_colmajor", [r, c],
                  2 * r * c + r * c + shape[0] * shape[1] * 4,
                  lambda a=a, q=qT3, s=sT3, f=pc: pq.qcast_per_channel_T_sf(
                      a, "e4m3", 128, sf_flags=f, out=q, out_sf=s)))
    r, n = wl.rows, wl.cols
    shape, dt = pq.sf_layout_shape(r, 2 * n, 128, pc)
    qb3 = torch.empty(r, 2 * n, dtype=torch.float8_e4m3fn, device=dev)
    sb3 = torch.empty(shape, dtype=dt, device=dev)
    calls.append(("swiglu_backward_ue8m0_colmajor", [r, 2 * n],
                  r * 2 * n * 2 + r * n * 2 + r * 4 + r * 2 * n + shape[0] * shape[1] * 4,
                  lambda hg=hg, dvg=dvg, wg=wg, q=qb3, s=sb3, f=pc:
                  pq.qcast_swiglu_backward_per_token_sf(hg, dvg, wg, "e4m3", 128, sf_flags=f,
                                                        swiglu_clamp=6.0, out=q, out_sf=s)))
    # per-token cast with 1 x 32 groups and fp32 column-major scales
    x = by["per_token"].x.to(dev)
    r, c = x.shape
    cm = pq.SF_COL_MAJOR
    shape, dt = pq.sf_layout_shape(r, c, 32, cm)
    qo2 = torch.empty(r, c, dtype=torch.float8_e4m3fn, device=dev)
    so2 = torch.empty(shape, dtype=dt, device=dev)
    calls.append(("per_token_f32_colmajor_g32", [r, c], 2 * r * c + r * c + r * (c // 32) * 4,
                  lambda x=x, qo=qo2, so=so2, f=cm: pq.qcast_per_token_sf(x, "e4m3", 32,
                                                                         sf_flags=f, out=qo,
                                                                         out_sf=so)))
    return calls


def time_extras(extras, dev, steps, warmup, min_launches=10):
    import torch
    for _ in range(warmup):
        for *_, fn in extras:
            fn()
    torch.cuda.synchronize()
    hev = HipEvents()
    # the same one-timed-launch-per-pass rotation as the step, over enough
    # passes to time every cast at least 10 times
    passes = max(steps, min_launches * len(extras))
    ev = make_events(hev, len(extras), passes)
    timed_runs([fn for *_, fn in extras], ev)
    ms_all = collect(ev, hev)
    out = {}
    for (name, shape, b, _), ms in zip(extras, ms_all):
        avg = sum(ms) / len(ms)
        out[name] = {"shape": shape, "bytes": b, "timed_launches": len(ms),
                     "avg_us": round(avg * 1e3, 2), **spread_us(ms),
                     "GBps": round(b / (avg * 1e-3) / 1e9, 1),
                     "frac": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    return out


def copy_ceilings(dev, sizes, runs=11):
    """Copies moving each byte count in `sizes` in total (half read, half
    written), each after a 1 GiB flush, median of `runs` - 1 timed runs
    (the first is dropped). Returns {nbytes: {...}} in GB/s:
      "library": the library's streaming copy (include/qcast_bench.h), timed
                 by events its own dispatch records, like the casts;
      "library_marker", "runtime_marker": the library copy and the HIP
                 runtime's device-to-device hipMemcpyAsync (torch's copy_
                 between two same-device tensors), both timed by events
                 recorded on the stream around the call, so that the two
                 copies are compared with the same timing method: the
                 runtime's copy is a ceiling that owes nothing to this
                 library."""
    import torch
    import precision_quantization_amd as pq
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    hev = HipEvents()
    out = {}
    for nbytes in sorted(set(sizes)):
        half = nbytes // 2 // 16 * 16
        src = torch.empty(half, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty(half, dtype=torch.uint8, device=dev)
        times = {"library": [], "library_marker": [], "runtime_marker": []}
        for _ in range(runs):
            flush.fill_(0)
            a, b = hev.create(), hev.create()
            pq.qcast_bench_time_next(a, b)
            pq.qcast_bench_copy(src, dst)
            torch.cuda.synchronize()
            times["library"].append(hev.elapsed_ms(a, b))
            hev.destroy(a)
            hev.destroy(b)
            for name, fn in (("library_marker", lambda: pq.qcast_bench_copy(src, dst)),
                             ("runtime_marker", lambda: dst.copy_(src))):
                flush.fill_(0)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                torch.cuda.synchronize()
                times[name].append(e0.elapsed_time(e1))
        out[nbytes] = {}
        for name, t in times.items():
            ms = sorted(t[1:])[len(t[1:]) // 2]
            out[nbytes][name] = 2 * half / (ms * 1e-3) / 1e9
        del src, dst
    return out


def _oracle_cast(name, xb, w):
    """One oracle call of the named step cast on bf16 bits xb (and weights w)."""
    import oracle
    if name == "per_token":
        oracle.per_token(xb, "e4m3", 128)
    elif name == "swiglu":
        oracle.swiglu_per_token(xb, w, "e4m3", 128)
    elif name == "per_block":
        oracle.per_block(xb, "e4m3", 128)
    elif name == "per_channel_T":
        oracle.per_channel_T(xb, "e4m3", 128)
    elif name == "e2m1":
        oracle.e2m1(xb, 32)


def flushed_runs(fns, dev, runs=30):
    """Each closure timed on `runs` dispatches, every one after a 1 GiB flush
    on the same stream (the cold-cache protocol), the closures interleaved;
    per closure the sorted durations in ms."""
    import torch
    import precision_quantization_amd as pq
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    hev = HipEvents()
    out = [[] for _ in fns]
    for r in range(runs):
        for i, fn in enumerate(fns):
            flush.fill_(r & 0xFF)
            a, b = hev.create(), hev.create()
            pq.qcast_bench_time_next(a, b)
            fn()
            torch.cuda.synchronize()
            out[i].append(hev.elapsed_ms(a, b))
            hev.destroy(a)
            hev.destroy(b)
    return [sorted(t) for t in out]


def pattern_ceiling(dev, x, runs=6):
    """The transposed per-channel cast against its memory traffic alone
    (include/qcast_bench.h: the same loads and qT stores, no arithmetic), on
    the cast's input x, the two alternating, each after a 1 GiB flush;
    medians of 5 timed runs each, in us: (traffic alone, the cast)."""
    import torch
    import precision_quantization_amd as pq
    rows, cols = x.shape
    out = torch.empty(cols, rows, dtype=torch.uint8, device=dev)
    q = torch.empty(cols, rows, dtype=torch.float8_e4m3fn, device=dev)
    sf = torch.empty(cols, rows // 128, dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    hev = HipEvents()
    times = ([], [])
    for _ in range(runs):
        for i in range(2):
            flush.fill_(0)
            a, b = hev.create(), hev.create()
            pq.qcast_bench_time_next(a, b)
            if i == 0:
                pq.qcast_bench_per_channel_T_traffic(x, out=out)
            else:
                pq.qcast_per_channel_T(x, "e4m3", 128, out=q, out_sf=sf)
            torch.cuda.synchronize()
            times[i].append(hev.elapsed_ms(a, b))
            hev.destroy(a)
            hev.destroy(b)
    med = [sorted(t[1:])[len(t[1:]) // 2] * 1e3 for t in times]
    return med[0], med[1]


def cpu_baseline(wls, fraction=1.0):
    """The oracle, single-threaded, on the first `fraction` of the rows of
    every workload (all of them by default: about 10 s of CPU work); GB/s
    over the same algorithmic bytes."""
    from precision_quantization_amd import workloads as W
    total_bytes = 0
    total_s = 0.0
    for name, wl in wls:
        n = max(128, int(wl.rows * fraction) // 128 * 128)
        sub = W.Workload(wl.name, wl.op, wl.x[:n], wl.fmt, wl.group,
                         w=None if wl.w is None else wl.w[:n])
        xb = W.bf16_bits(sub.x)
        w = None if sub.w is None else sub.w.numpy()
        t0 = time.perf_counter()
        _oracle_cast(name, xb, w)
        total_s += time.perf_counter() - t0
        total_bytes += sub.algorithmic_bytes()
    return total_bytes / total_s / 1e9, total_s


def cpu_baseline_all_cores(wls, max_threads=16):
    """The same oracle calls over a static split of every workload's rows
    into whole 128-row parts, one Python thread per part on the cores this
    process may use (at most max_threads; the oracle's C calls release the
    GIL); GB/s over the same algorithmic bytes, and the threads used."""
    import threading
    from precision_quantization_amd import workloads as W
    nthreads = max(1, min(max_threads, len(os.sched_getaffinity(0))))
    total_bytes = 0
    total_s = 0.0
    for name, wl in wls:
        xb = W.bf16_bits(wl.x)
        w = None if wl.w is None else wl.w.numpy()
        groups = wl.rows // 128
        parts = min(nthreads, groups)
        bounds = [128 * (groups * i // parts) for i in range(parts + 1)]
        threads = [threading.Thread(target=_oracle_cast,
                                    args=(name, xb[a:b], None if w is None else w[a:b]))
                   for a, b in zip(bounds[:-1], bounds[1:])]
        t0 = time.perf_counter()
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        total_s += time.perf_counter() - t0
        total_bytes += wl.algorithmic_bytes()
    return total_bytes / total_s / 1e9, total_s, nthreads


def load_traffic(dominant):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, if it was taken from the library as it is now built."""
    try:
        from precision_quantization_amd import build
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("library_digest") != build.source_digest():
            return None
        return t["kernels"][dominant]["bytes_per_launch"]
    except (OSError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip timing the casts that are not part of the step")
    ap.add_argument("--profile-run", action="store_true",
                    help="every kernel, each timing loop cut to a few launches: for the "
                         "counter passes of rocprofv3, where every dispatch is slow")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0:
        ap.error("--steps must be at least 1 and --warmup at least 0")
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the casts shard "
              "by rows with no exchange between GPUs, so a multi-GPU run adds nothing to "
              "measure here.", file=sys.stderr)
        sys.exit(2)

    import torch
    from precision_quantization_amd import workloads as W
    dev = torch.device("cuda:0")
    log("bench: generating workloads")
    wls = make_workloads()
    calls = kernel_calls(wls, dev)
    step_bytes = sum(wl.algorithmic_bytes() for _, wl in wls)
    torch.cuda.synchronize()
    log("bench: warmup")
    for _ in range(args.warmup):
        for _, _, fn in calls:
            fn()
    torch.cuda.synchronize()

    fns = [fn for _, _, fn in calls]
    log(f"bench: timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for fn in fns:
            fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    # per-kernel durations: after the headline loop and outside `value`,
    # steps in which kernel s mod n records events from its own dispatch,
    # enough of them for every kernel to be timed MIN_TIMED_LAUNCHES times
    hev = HipEvents()
    min_launches = 0 if args.profile_run else MIN_TIMED_LAUNCHES
    rot_steps = max(args.steps, min_launches * len(fns))
    log(f"bench: per-kernel timing over {rot_steps} steps")
    ev = make_events(hev, len(fns), rot_steps)
    timed_runs(fns, ev)

    kernels = {}
    for (name, wl, _), ms in zip(calls, collect(ev, hev)):
        avg = sum(ms) / len(ms)
        b = wl.algorithmic_bytes()
        kernels[name] = {
            "shape": list(wl.x.shape), "bytes": b, "timed_launches": len(ms),
            "avg_us": round(avg * 1e3, 2), **spread_us(ms),
            "GBps": round(b / (avg * 1e-3) / 1e9, 1),
            "frac": round(b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "rows_per_s": round(wl.rows / (avg * 1e-3)),
            "input_sha256": W.sha256(wl.x),
        }
        if getattr(wl, "w", None) is not None:
            kernels[name]["weight_sha256"] = W.sha256(wl.w)
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    d = kernels[dominant]
    traffic = load_traffic(dominant)
    # the largest size last, so the copy the counter runs calibrate on is the
    # last copy of the run
    copy_nbytes = max(k["bytes"] for k in kernels.values())
    log("bench: copy ceilings (library copy and the runtime's hipMemcpyAsync)")
    reps = 2 if args.profile_run else None
    ceilings = copy_ceilings(dev, [k["bytes"] for k in kernels.values()], runs=reps or 11)
    copy_gbs = ceilings[copy_nbytes]["library"]
    for k in kernels.values():
        c = ceilings[k["bytes"]]
        k["copy_GBps"] = round(c["library"], 1)
        k["of_copy"] = round(k["GBps"] / c["library"], 4)
        k["runtime_copy_GBps"] = round(c["runtime_marker"], 1)
        k["library_copy_marker_GBps"] = round(c["library_marker"], 1)
    for (name, wl, _), ms in zip(calls, flushed_runs([fn for _, _, fn in calls], dev,
                                                     runs=reps or 30)):
        k = kernels[name]
        sp = spread_us(ms)
        k["flushed"] = {"runs": len(ms), "median_us": sp["median_us"], "p10_us": sp["p10_us"],
                        "p90_us": sp["p90_us"],
                        "GBps": round(k["bytes"] / (sp["median_us"] * 1e-6) / 1e9, 1)}
    pt = kernels["per_channel_T"]
    pc_x = next(wl for name, wl in wls if name == "per_channel_T").x.to(dev)
    pattern_us, flushed_us = pattern_ceiling(dev, pc_x, runs=reps or 6)
    pt["pattern_us"] = round(pattern_us, 2)
    pt["flushed_us"] = round(flushed_us, 2)
    pt["of_pattern"] = round(pattern_us / flushed_us, 4)
    del pc_x
    result = {
        "metric": METRIC,
        "value": round(step_bytes * args.steps / elapsed / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "one pass of the five casts on DeepSeek-V3-shaped inputs: per_token "
                        "X[4096,7168] E4M3 g128; swiglu H[8192,4096]+w E4M3 g128; per_block "
                        "W[7168,18432] E4M3 128x128; per_channel_T A[16384,7168] E4M3 g128 "
                        "transposed; e2m1 X[16384,7168] packed g32",
            "step_bytes": step_bytes,
        },
        "roofline": {
            "bound": "hbm", "kernel": dominant, "achieved": d["GBps"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": d["frac"], "traffic": traffic,
        },
        "kernels": kernels,
        "copy_ceiling_GBps": round(copy_gbs, 1),
        "copy_bytes": copy_nbytes // 2 // 16 * 16 * 2,
        "runtime_copy_ceiling_GBps": round(ceilings[copy_nbytes]["runtime_marker"], 1),
        "library_copy_marker_GBps": round(ceilings[copy_nbytes]["library_marker"], 1),
    }
    if not args.no_extras:
        log("bench: timing the other casts")
        result["other_kernels"] = time_extras(extra_calls(wls, dev), dev, args.steps,
                                              args.warmup,
                                              min_launches=0 if args.profile_run else 10)
    if not args.no_cpu_baseline:
        log("bench: CPU baseline (oracle)")
        gbs, secs = cpu_baseline(wls)
        result["cpu_baseline"] = {
            "value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"all rows of each of the five workloads, one oracle call each "
                      f"({secs:.1f} s on {cpu_model()}, "
                      f"{os.cpu_count()} cores present)",
        }
        log("bench: CPU baseline over all cores (oracle)")
        gbs_n, secs_n, threads = cpu_baseline_all_cores(wls)
        result["cpu_baseline_all_cores"] = {
            "value": round(gbs_n, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"all rows of each of the five workloads, split into {threads} parts of "
                      f"whole 128-row groups, one thread each ({secs_n:.1f} s)",
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
