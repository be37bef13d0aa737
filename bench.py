"""Benchmark of the MXFP4 MoE expert path on one MI355X.

A step is one pass of the whole path over one batch: activation quantisation,
routing + permutation, the grouped FC1 (+ fused SwiGLU / requantisation) and
FC2 GEMMs, and the gate-weighted combine - all on device-resident inputs.

Headline workload: the 16384-token prefill layer with FP4 x FP4 products
(hidden 7168, intermediate 2048, 256 experts, top-6, MXFP4 activations),
value = algorithmic TFLOP/s of the layer (pairs x 88,080,384 flop / step time).
Also reported on the same line: the 8-token decode layer (weight GB/s over the
touched experts), the 2048-token Zipf-routed FP8 layer (TFLOP/s and touched-weight
GB/s), the dense 64 x 4096 x 7168 and 16 x 32 x 4096 GEMMs, and the FP4-weight GEMM
variants (bf16 activations with MXFP4 / NVFP4 weights, Q8 lookup-table route), each
against its roofline.
The fp64 CPU oracle is timed on a bounded sample of the headline workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
                       [--only prefill|decode|dense|skewed|variants|copy|calib]

--only calib runs the dense E2M1 GEMM 256 x 8192 x 7168 per step (no JSON line): an
LDS-DMA kernel whose HBM reads are known, to check the FETCH_SIZE scale factor.
--only copy runs a plain device-to-device copy of 1 GiB per step (no JSON line):
the reference kernel of known byte count that scales the FETCH_SIZE / WRITE_SIZE
hardware counters into HBM bytes.
"""

import argparse
import json
import subprocess
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mxfp4_block_scaled_amd import datagen as dg  # noqa: E402
from mxfp4_block_scaled_amd import ops  # noqa: E402

METRIC = "MoE MXFP4 grouped-GEMM TFLOP/s (prefill) & weight GB/s (decode) vs roofline"
PEAK_HBM_GBS = 8000.0
# bytes the probe's stage moves into LDS; the 256 x 256 FP4 ring kernel's stage moves 64 KB
# of codes plus 4 KB of scales (a 16 KB scale group every 4 stages)
LDS_FILL_STAGE_BYTES = 65536
RING_STAGE_BYTES = 65536 + 4096
PEAK_TFLOPS = {"e2m1": 10100.0, "e4m3": 5000.0}  # dense MXFP4 / MXFP8 (FP8 x FP4 runs at the FP8 rate)
FLOP_PER_PAIR = 2 * 7168 * 4096 + 2 * 2048 * 7168  # 88,080,384
BYTES_PER_EXPERT = 4096 * 3584 + 4096 * 224 + 7168 * 1024 + 7168 * 64  # 23,396,352

# HBM bytes per grouped-GEMM call (its FC1 + FC2 launches; "_fused": FC1 + the fused FC2 and
# combine) from rocprofv3 FETCH_SIZE / WRITE_SIZE passes, scaled by a 1 GiB copy (2.0 x
# FETCH_SIZE + 1.0 x WRITE_SIZE, checked on an LDS-DMA GEMM of known bytes; the passes and the
# calibration are in profiles/moe_layer_hbm_traffic.md). They hold only for the GEMM sources
# they were measured on (sha-256 over GEMM_SOURCES): on any other source traffic = null.
TRAFFIC_SRC_SHA256 = "3a7190cdea46bb71ff62cb93561c5f3ff45b76bcf51056a30bc9c9514ae3f104"
TRAFFIC_BYTES = {"moe_prefill_t16384_fp4": 8861863526, "moe_decode_t8_fused": 1022578995,
                 "moe_decode_t8": 1008449229, "moe_prefill_t2048_zipf": 3164287283}


GEMM_SOURCES = ("gemm.hip", "gemm_common.hpp", "gemm_stream.hip", "gemm_tile.hip", "gemm_wide.hip", "gemm_f8ring.hip",
                "tile256.hpp", "mx_codec.hpp", "fc2_combine.hip")


def gemm_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mxfp4_block_scaled_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload):
    if gemm_sources_sha256() != TRAFFIC_SRC_SHA256:
        return None
    return TRAFFIC_BYTES.get(workload)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def moe_weights_dev(cfg):
    """All experts' weights, generated expert by expert straight into device tensors."""
    E, H, I = cfg["E"], cfg["H"], cfg["I"]
    w1 = torch.empty((E, 2 * I, H // 2), dtype=torch.uint8, device="cuda")
    s1 = torch.empty((E, 2 * I, H // 32), dtype=torch.uint8, device="cuda")
    w2 = torch.empty((E, H, I // 2), dtype=torch.uint8, device="cuda")
    s2 = torch.empty((E, H, I // 32), dtype=torch.uint8, device="cuda")
    for e in range(E):
        parts = dg.expert_weights(cfg["seed"], e, H, I, cfg["exp_lo"], cfg["exp_hi"])
        for dst, src in zip((w1, s1, w2, s2), parts):
            dst[e].copy_(torch.from_numpy(src), non_blocking=False)
    return w1, s1, w2, s2


class Layer:
    """Pre-allocated buffers of one MoE layer; step() = the four C-ABI calls, or with
    fused=True (at most 64 tokens) two: quantisation with routing, and both FCs with
    FC2 fused into the combine."""

    def __init__(self, cfg, weights_sets, y_dtype=torch.bfloat16, fused=False):
        self.cfg = cfg
        T, H, I, k = cfg["T"], cfg["H"], cfg["I"], cfg["k"]
        self.fmt = cfg["act_fmt"]
        self.x = bf16_dev(dg.activations(cfg["seed"], T, H))
        self.logits = to_dev(dg.logits(cfg["seed"], T, cfg["E"], cfg["routing"]))
        self.sets = weights_sets
        self.y_dtype = y_dtype
        self.fused = fused
        self.T, self.k = T, k
        R = T * k
        fp4 = self.fmt == "e2m1"
        self.q = torch.empty((T, H // 2 if fp4 else H), dtype=torch.uint8, device="cuda")
        self.qs = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
        self.ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        self.gates = torch.empty((T, k), dtype=torch.float32, device="cuda")
        self.offs = torch.empty((cfg["E"] + 1,), dtype=torch.int32, device="cuda")
        self.sp = torch.empty((R,), dtype=torch.int32, device="cuda")
        self.pr = torch.empty((R,), dtype=torch.int32, device="cuda")
        self.h = torch.empty((R, I // 2 if fp4 else I), dtype=torch.uint8, device="cuda")
        self.hs = torch.empty((R, I // 32), dtype=torch.uint8, device="cuda")
        self.y = torch.empty((R, H), dtype=y_dtype, device="cuda")
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        self.lib = ops.load()
        self.i = 0

    def step(self, ev=None):
        c, lib = self.cfg, self.lib
        st = ctypes_stream()
        P = ops._ptr
        w1, s1, w2, s2 = self.sets[self.i % len(self.sets)]
        self.i += 1
        f = ops.FMTS[self.fmt]
        if ev: ev[0].record()
        if self.fused:
            ops._check(lib.moe_quantize_route(P(self.x), ops.MXF_BF16, P(self.logits), self.T, c["H"], c["E"],
                                              self.k, f, P(self.q), P(self.qs), P(self.ids), P(self.gates),
                                              P(self.offs), P(self.sp), P(self.pr), st), "quantize+route")
            if ev:
                ev[1].record()
                ev[2].record()
        else:
            ops._check(lib.mxfp4_quantize_act(P(self.x), ops.MXF_BF16, self.T, c["H"], f, P(self.q), P(self.qs),
                                              st), "quantize")
            if ev: ev[1].record()
            ops._check(lib.moe_route_permute(P(self.logits), self.T, c["E"], self.k, P(self.ids), P(self.gates),
                                             P(self.offs), P(self.sp), P(self.pr), st), "route")
            if ev: ev[2].record()
        if self.fused:
            ops._check(lib.moe_grouped_mxfp4_gemm_combine(
                P(self.q), P(self.qs), f, self.T, self.k, c["H"], c["I"], c["E"], P(self.offs), P(self.sp),
                P(self.ids), P(self.pr), P(self.gates), P(w1), P(s1), P(w2), P(s2), P(self.h), P(self.hs), P(self.out), ops.MXF_BF16, st),
                "grouped+combine")
            if ev:
                ev[3].record()
                ev[4].record()
            return
        ops._check(lib.moe_grouped_mxfp4_gemm(P(self.q), P(self.qs), f, self.T, self.k, c["H"], c["I"], c["E"],
                                              P(self.offs), P(self.sp), P(w1), P(s1), P(w2), P(s2), P(self.h),
                                              P(self.hs), P(self.y), ops.DTYPES[self.y_dtype], st), "grouped")
        if ev: ev[3].record()
        ops._check(lib.moe_unpermute_combine(P(self.y), ops.DTYPES[self.y_dtype], P(self.gates), P(self.pr),
                                             self.T, self.k, c["H"], P(self.out), ops.MXF_BF16, st), "combine")
        if ev: ev[4].record()


KERNEL_TIMES = True  # set from --no-kernel-times


def kernel_times_us(step_fn, reps=3):
    """Mean device time per step of each kernel, from torch's profiler (a separate,
    untimed pass; {} if the profiler is unavailable or switched off)."""
    if not KERNEL_TIMES:
        return {}
    try:
        from torch.profiler import ProfilerActivity, profile
        step_fn(None)
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CUDA]) as prof:
            for _ in range(reps):
                step_fn(None)
            torch.cuda.synchronize()
        out = {}
        for ev in prof.key_averages():
            t = getattr(ev, "device_time_total", None)
            if t is None:
                t = getattr(ev, "cuda_time_total", 0.0)
            if t and "mxf::" in ev.key:
                out[ev.key] = out.get(ev.key, 0.0) + t / reps
        return out
    except Exception as ex:  # the report stays valid without it
        log(f"[bench] kernel times unavailable: {ex}")
        return {}


def pick(times, *needles):
    """Sum of the kernel times whose names contain every needle."""
    v = sum(t for k, t in times.items() if all(n in k for n in needles))
    return round(v, 2) if v else None


def gpu_clocks():
    """Current clocks as rocm-smi reports them (None if it cannot be run, and not
    asked for in runs under an outside profiler: --no-kernel-times)."""
    if not KERNEL_TIMES:
        return None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        return {k.strip(" :"): v for k, v in card.items() if "clk" in k.lower()}
    except Exception:
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def ctypes_stream():
    import ctypes
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def time_steps(step_fn, steps, warmup, nev=0):
    for _ in range(warmup):
        step_fn(None)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)] if nev else None
    t0 = time.perf_counter()
    for i in range(steps):
        step_fn(evs[i] if evs else None)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    stages = None
    if evs:
        stages = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nev - 1)] for i in range(steps)])
    return wall, stages


def time_graph_steps(layer, steps, warmup):
    """The same step captured once per weight set in a HIP graph (the library
    allocates and synchronises nothing, so a whole step captures) and replayed in
    rotation: what a serving loop that replays its decode step pays per step."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.step(None)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graphs = []
    for j in range(len(layer.sets)):
        layer.i = j
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.step(None)
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def bench_moe(name, steps, warmup, rotate, fused=False, sets=None):
    cfg = dg.WORKLOADS[name]
    if sets is None:
        log(f"[bench] {name}: generating inputs ...")
        t0 = time.time()
        base = moe_weights_dev(cfg)
        sets = [base] + [tuple(t.clone() for t in base) for _ in range(rotate - 1)]
        log(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s ({rotate} weight set(s))")
    layer = Layer(cfg, sets, fused=fused)
    # the step's wall time from a loop without timing events (their markers add gaps
    # between kernels), then the per-stage times from a second loop with events
    wall, _ = time_steps(layer.step, steps, warmup)
    _, st = time_steps(layer.step, steps, 1, nev=5)
    names = ["quantize", "route_permute", "grouped_gemm", "combine"]
    if fused:
        names = ["quantize_route", None, "grouped_gemm_combine"]  # one launch for the first two
    stage_ms = {n: float(np.mean(st[:, j])) for j, n in enumerate(names) if n}
    offs = layer.offs.cpu().numpy()
    counts = np.diff(offs)
    touched = int((counts > 0).sum())
    pairs = cfg["T"] * cfg["k"]
    flops = pairs * FLOP_PER_PAIR
    wbytes = touched * BYTES_PER_EXPERT
    return dict(cfg=cfg, ms=wall * 1e3, stage_ms=stage_ms, touched=touched, pairs=pairs, flops=flops,
                wbytes=wbytes, max_rows=int(counts.max()), units256=int(((counts + 255) // 256).sum()),
                layer=layer, sets=sets)


def bench_dense(steps, warmup, rotate=48, name="dense_m64_n4096_k7168"):
    cfg = dg.WORKLOADS[name]
    d = dg.workload_inputs(name)
    a = bf16_dev(d["a"])
    w0, s0 = to_dev(d["w"]), to_dev(d["w_scale"])
    sets = [(w0, s0)] + [(w0.clone(), s0.clone()) for _ in range(rotate - 1)]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    lib = ops.load()
    ws = torch.empty(lib.mxfp4_gemm_workspace_bytes(M, N, K, 0), dtype=torch.uint8, device="cuda")
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    it = [0]

    def step(ev):
        w, s = sets[it[0] % len(sets)]
        it[0] += 1
        if ev: ev[0].record()
        ops._check(lib.mxfp4_gemm(ops._ptr(a), M, N, K, 0, ops._ptr(w), ops._ptr(s), ops._ptr(c), ops._ptr(ws),
                                  ws.numel(), ctypes_stream()), "mxfp4_gemm")
        if ev: ev[1].record()

    wall, st = time_steps(step, steps * 10, warmup, nev=2)
    ms = float(np.mean(st[:, 0]))
    # the same calls back to back from one HIP graph (one call per weight set)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(None)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(len(sets)):
            step(None)
    for _ in range(max(warmup, 1)):
        g.replay()
    torch.cuda.synchronize()
    reps = max(steps // 4, 2)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) / (reps * len(sets)) * 1e3
    wbytes = N * K // 2 + N * K // 32
    return dict(ms=ms, graph_ms=graph_ms, wbytes=wbytes, gbs=wbytes / (ms * 1e-3) / 1e9, flops=2 * M * N * K)


def bench_fp4_variants(steps, warmup, rotate=48):
    """The FP4-weight GEMMs beside the MX path at the pages' accuracy-table shapes:
    bf16 activations with MXFP4 or NVFP4 weights, and the lookup-table route (Q8
    activations, int8-expanded MXFP4 weights; its activation quantisation timed on its
    own). Weight sets rotate (48 x ~15 MB, beyond the 256 MB cache) so the weights come
    from HBM; value = weight (+ scale) bytes / call time."""
    lib = ops.load()
    out = {}
    for (M, N, K) in ((1, 4096, 7168), (64, 4096, 7168)):
        x = bf16_dev(dg.activations(7, M, K, outliers=True))
        mw, ms = dg.dense_weights(7, N, K, 120, 128)
        nw, ns = dg.nvfp4_weights(7, N, K)
        mx = [(to_dev(mw), to_dev(ms))] * 1
        mx += [(mx[0][0].clone(), mx[0][1].clone()) for _ in range(rotate - 1)]
        nv = [(to_dev(nw), to_dev(ns))]
        nv += [(nv[0][0].clone(), nv[0][1].clone()) for _ in range(rotate - 1)]
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(lib.fp4_w4a16_workspace_bytes(M, N, K), 1), dtype=torch.uint8, device="cuda")
        q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        dq = torch.empty((M, K // 32), dtype=torch.float16, device="cuda")
        P = ops._ptr
        it = [0]

        def run(fn, sets):
            def step(ev):
                w, s_ = sets[it[0] % len(sets)]
                it[0] += 1
                if ev: ev[0].record()
                ops._check(fn(w, s_), "fp4 variant")
                if ev: ev[1].record()
            _, st = time_steps(step, steps * 10, warmup, nev=2)
            return float(np.mean(st[:, 0]))

        st = ctypes_stream()
        ms_w16 = run(lambda w, s_: lib.mxfp4_gemm_w4a16(P(x), M, N, K, P(w), P(s_), P(c), P(ws), ws.numel(), st), mx)
        ms_nv = run(lambda w, s_: lib.nvfp4_gemm_w4a16(P(x), M, N, K, P(w), P(s_), P(c), P(ws), ws.numel(), st), nv)
        ms_qa = run(lambda w, s_: lib.q8_quantize_act(P(x), M, K, P(q), P(dq), st), mx)
        ms_q8 = run(lambda w, s_: lib.mxfp4_gemm_q8(P(q), P(dq), M, N, K, P(w), P(s_), P(c), P(ws), ws.numel(), st),
                    mx)
        mxb, nvb = N * K // 2 + N * K // 32, N * K // 2 + N * K // 16
        key = f"m{M}_n{N}_k{K}"
        out[key] = {
            "w4a16_mxfp4": {"us": round(ms_w16 * 1e3, 2), "weight_GBps": round(mxb / (ms_w16 * 1e-3) / 1e9, 1),
                            "frac_hbm": round(mxb / (ms_w16 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "w4a16_nvfp4": {"us": round(ms_nv * 1e3, 2), "weight_GBps": round(nvb / (ms_nv * 1e-3) / 1e9, 1),
                            "frac_hbm": round(nvb / (ms_nv * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
            "q8_lut": {"us": round(ms_q8 * 1e3, 2), "quantize_us": round(ms_qa * 1e3, 2),
                       "weight_GBps": round(mxb / (ms_q8 * 1e-3) / 1e9, 1),
                       "frac_hbm": round(mxb / (ms_q8 * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        }
        del mx, nv
        torch.cuda.empty_cache()
    return out


def measure_ceilings(reps=3):
    """What this GPU sustains for the bounds (include/mxf_ceilings.h), best of `reps`:
    a non-temporal streaming read of 2 GiB, register-only loops of 32x32x64 scaled
    MFMAs on random operand bits (E2M1 x E2M1, E4M3 x E2M1), and the HBM -> LDS copy
    path alone (own bytes / the FC1 launch's sharing)."""
    lib = ops.load()
    st = ctypes_stream()
    buf = torch.ones(1 << 29, dtype=torch.int32, device="cuda")  # 2 GiB
    xo = torch.zeros(1, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(17)
    words = torch.randint(-2**31, 2**31 - 1, (ops.CEILING_MFMA_WORDS,), dtype=torch.int32, device="cuda",
                          generator=g)
    sink = torch.empty(ops.CEILING_MFMA_GROUPS, dtype=torch.float32, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        t = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            t.append(e0.elapsed_time(e1))
        return min(t)

    nbytes = buf.numel() * 4
    ms_read = best(lambda: ops._check(lib.mxf_ceiling_read(ops._ptr(buf), nbytes, ops._ptr(xo), st), "read"))
    iters = 20000
    flops = lib.mxf_ceiling_mfma_flops(iters)
    out = {"hbm_read_GBps": round(nbytes / (ms_read * 1e-3) / 1e9, 1)}
    for key, f in (("mfma_e2m1_random_TFLOPs", ops.MXF_E2M1), ("mfma_e4m3xe2m1_random_TFLOPs", ops.MXF_E4M3)):
        ms = best(lambda: ops._check(lib.mxf_ceiling_mfma(f, ops._ptr(words), words.numel(), 124, iters,
                                                          ops._ptr(sink), st), "mfma"))
        out[key] = round(flops / (ms * 1e-3) / 1e12, 1)
    # the prefill GEMMs' operand copies on their own: 28 stages of 64 KB into LDS per
    # workgroup, each workgroup reading its own bytes (HBM streaming) or sharing them as
    # the grouped FC1 launch does (16 workgroups per activation unit, 2 per weight tile)
    sm = torch.zeros(1, dtype=torch.int32, device="cuda")
    for key, pattern, groups in (("lds_fill_own_GBps", 0, 1024), ("lds_fill_fc1_sharing_GBps", 1, 2048)):
        assert lib.mxf_ceiling_lds_copy_bytes(pattern, groups) <= nbytes
        ms = best(lambda: ops._check(lib.mxf_ceiling_lds_copy(ops._ptr(buf), nbytes, pattern, groups, ops._ptr(sm),
                                                              st), "lds_copy"))
        out[key] = round(groups * LDS_FILL_STAGE_BYTES * ops.CEILING_COPY_STAGES / (ms * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return out


def cpu_baseline(name, budget_s=15.0):
    """The fp64 oracle (as it stands) on a bounded sample: whole experts of the
    headline layer, all their rows, until ~budget_s of CPU time is spent."""
    import oracle
    from threadpoolctl import threadpool_info

    cfg = dg.WORKLOADS[name]
    T, H, I, k, E = cfg["T"], cfg["H"], cfg["I"], cfg["k"], cfg["E"]
    x = dg.activations(cfg["seed"], T, H)
    logits = dg.logits(cfg["seed"], T, E, cfg["routing"])
    fmt = cfg["act_fmt"]
    t0 = time.perf_counter()
    q, qs = oracle.moe.quantize_act(oracle.bf16_bits_to_f64(x), fmt)
    ids, gates = oracle.route_topk(logits, k)
    offs, sp, pr = oracle.permute(ids, E)
    t_pre = time.perf_counter() - t0
    done_pairs, t_gemm, e = 0, 0.0, 0
    while e < E and (t_gemm < budget_s or e == 0):
        w1, s1, w2, s2 = dg.expert_weights(cfg["seed"], e, H, I, cfg["exp_lo"], cfg["exp_hi"])
        rows = np.arange(offs[e], offs[e + 1])
        t1 = time.perf_counter()
        tok = sp[rows] // k
        a_hat = oracle.moe.decode_act(q[tok], qs[tok], fmt)
        G, hp = oracle.fc1_swiglu_rows(a_hat, w1, s1, I)
        hq, hs = oracle.moe.quantize_act(hp, fmt)
        oracle.fc2_rows(hq, hs, fmt, w2, s2)
        t_gemm += time.perf_counter() - t1
        done_pairs += rows.size
        e += 1
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tflops = done_pairs * FLOP_PER_PAIR / t_gemm / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{name}: quantize+route+permute of all {T} tokens ({t_pre:.1f}s), then FC1+SwiGLU+"
                      f"requantise+FC2 in fp64 for experts 0..{e - 1} ({done_pairs} pairs, {t_gemm:.1f}s); "
                      f"value = sampled pairs x 88,080,384 flop / FC time"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    # no torch.profiler pass for the per-kernel split (for runs under an outside profiler)
    ap.add_argument("--no-kernel-times", action="store_true")
    # one workload (or the copy reference kernel) instead of the default line
    ap.add_argument("--only", choices=["prefill", "decode", "dense", "skewed", "variants", "copy", "calib"],
                    default=None)
    # the achievable-rate probes run with the default line; with --only, on request
    ap.add_argument("--ceilings", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the expert path here is the "
              "single-GPU kernel; no multi-GPU figure is measured.", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    global KERNEL_TIMES
    KERNEL_TIMES = not args.no_kernel_times
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for i in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy: {args.warmup + args.steps} copies of {n} bytes")
        return
    if args.only == "calib":
        # an LDS-DMA kernel whose HBM reads are known: the dense E2M1 GEMM with one 256-row
        # unit (256 x 256 tiles, copies by buffer_load ... lds), where every weight tile is
        # read by one workgroup and the activation codes are shared through L2
        M, N, K = 256, 8192, 7168
        a = bf16_dev(dg.activations(5, M, K))
        w, s_ = (to_dev(t) for t in dg.dense_weights(5, N, K, 120, 128))
        lib = ops.load()
        ws = torch.empty(lib.mxfp4_gemm_workspace_bytes(M, N, K, ops.MXF_E2M1), dtype=torch.uint8, device="cuda")
        c = torch.empty((M, N), dtype=torch.float32, device="cuda")
        for i in range(args.warmup + args.steps):
            ops.mxfp4_gemm(a, w, s_, "e2m1", out=c, workspace=ws)
        torch.cuda.synchronize()
        reads = N * K // 2 + N * K // 32 + M * K // 2 + M * K // 32
        log(f"[bench] calib: {args.warmup + args.steps} dense E2M1 GEMMs {M}x{N}x{K}; the GEMM kernel reads "
            f"{reads} bytes (weights, their scales, activation codes and scales, each once) and writes {M * N * 4}")
        return
    ops.load()
    torch.cuda.synchronize()
    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic"}

    ceil = measure_ceilings() if args.only is None or args.ceilings else None
    if ceil:
        result["ceilings"] = ceil
    if args.only in (None, "prefill"):
        name = "moe_prefill_t16384_fp4"
        r = bench_moe(name, args.steps, args.warmup, rotate=1)
        cfg = r["cfg"]
        tflops = r["flops"] / (r["ms"] * 1e-3) / 1e12
        g_ms = r["stage_ms"]["grouped_gemm"]
        g_tflops = r["flops"] / (g_ms * 1e-3) / 1e12
        peak = PEAK_TFLOPS[cfg["act_fmt"]]
        result.update({
            "value": round(tflops, 3), "unit": "TFLOP/s", "ms_per_step": round(r["ms"], 4),
            "dtype": "mxfp4 (e2m1 x e2m1, ue8m0 scales, fp32 accumulate)",
            "config": {"workload": name, "T": cfg["T"], "H": cfg["H"], "I": cfg["I"], "E": cfg["E"],
                       "topk": cfg["k"], "act_fmt": cfg["act_fmt"], "routing": cfg["routing"],
                       "seed": cfg["seed"], "pairs": r["pairs"], "max_rows_per_expert": r["max_rows"]},
            "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
            "roofline": {"kernel": "moe_grouped_mxfp4_gemm (FC1 + FC2 kernels)", "bound": "mfma",
                         "achieved": round(g_tflops, 3), "peak": peak, "unit": "TFLOP/s",
                         "frac": round(g_tflops / peak, 4), "traffic": measured_traffic(name)},
        })
        if ceil:
            result["frac_of_measured_ceiling"] = round(g_tflops / ceil["mfma_e2m1_random_TFLOPs"], 4)
        # FC1 and FC2 apart (the grouped-GEMM call launches both): device times per step
        # (the profiler's tracer lengthens these long kernels by 10-20 %, so its times give
        # the split of the event-timed grouped-GEMM stage, not the times themselves)
        kt = kernel_times_us(r["layer"].step)
        fc1, fc2 = pick(kt, "<0,"), pick(kt, "<1,")
        if fc1 and fc2:
            fl1, fl2 = r["pairs"] * 58720256, r["pairs"] * 29360128
            t1, t2 = g_ms * fc1 / (fc1 + fc2), g_ms * fc2 / (fc1 + fc2)
            result["fc1_fc2"] = {"fc1_ms": round(t1, 4), "fc2_ms": round(t2, 4),
                                 "fc1_TFLOPs": round(fl1 / t1 / 1e9, 1), "fc2_TFLOPs": round(fl2 / t2 / 1e9, 1),
                                 "fc1_frac": round(fl1 / t1 / 1e9 / peak, 4), "fc2_frac": round(fl2 / t2 / 1e9 / peak, 4),
                                 "profiler_us": {"fc1": fc1, "fc2": fc2},
                                 "method": "grouped_gemm stage time split by the FC1 / FC2 kernel-time ratio "
                                           "from torch.profiler (3 steps after the timed loops)"}
            # the copy path: bytes the ring kernels move into LDS per call (units x n-tiles x
            # stages x 68 KB) over each kernel's time, against the copy probe's rate
            u = r["units256"]
            b1 = u * (2 * cfg["I"] // 256) * (cfg["H"] // 256) * RING_STAGE_BYTES
            b2 = u * (cfg["H"] // 256) * (cfg["I"] // 256) * RING_STAGE_BYTES
            lf = {"units": u, "fc1_bytes": b1, "fc2_bytes": b2,
                  "fc1_GBps": round(b1 / t1 / 1e6, 1), "fc2_GBps": round(b2 / t2 / 1e6, 1)}
            if ceil:
                lf["fc1_frac_of_sharing_ceiling"] = round(b1 / t1 / 1e6 / ceil["lds_fill_fc1_sharing_GBps"], 4)
            result["lds_fill"] = lf
        result["gpu_clocks_after_prefill"] = gpu_clocks()
        del r["layer"], r["sets"]
        torch.cuda.empty_cache()
    if args.only in (None, "decode"):
        name = "moe_decode_t8"
        # the product's decode step: FC2 fused with the combine; the unfused four-call
        # step on the same weights beside it
        r = bench_moe(name, args.steps * 5, args.warmup, rotate=2, fused=True)
        u = bench_moe(name, args.steps * 5, args.warmup, rotate=2, sets=r["sets"])
        g_ms = r["stage_ms"]["grouped_gemm_combine"]
        gbs = lambda ms: round(r["wbytes"] / (ms * 1e-3) / 1e9, 1)
        dec = {"workload": name, "ms_per_step": round(r["ms"], 4),
               "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
               "touched_experts": r["touched"], "weight_bytes": r["wbytes"],
               "weight_GBps_layer": gbs(r["ms"]),
               "weight_GBps_grouped_gemm_combine": gbs(g_ms),
               "roofline": {"kernel": "moe_grouped_mxfp4_gemm_combine (FC1 + fused FC2/combine kernels)",
                            "bound": "hbm", "achieved": gbs(g_ms), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs(g_ms) / PEAK_HBM_GBS, 4),
                            "traffic": measured_traffic(name + "_fused")}}
        kt = kernel_times_us(r["layer"].step, reps=10)
        dec["kernels_us"] = {"quantize_route": pick(kt, "quantize_route_kernel"),
                             "fc1": pick(kt, "gemm_stream1_kernel", ", 0,"),
                             "fc2_combine": pick(kt, "fc2_combine_kernel"),
                             "source": "torch.profiler device times, 10 steps after the timed loops"}
        ug = u["stage_ms"]["grouped_gemm"]
        dec["unfused"] = {"ms_per_step": round(u["ms"], 4),
                          "stages_ms": {k: round(v, 4) for k, v in u["stage_ms"].items()},
                          "weight_GBps_layer": gbs(u["ms"]), "weight_GBps_grouped_gemm": gbs(ug),
                          "traffic_grouped_gemm": measured_traffic(name)}
        g_wall = time_graph_steps(r["layer"], args.steps * 5, args.warmup)
        if ceil:
            dec["frac_of_measured_ceiling"] = round(dec["roofline"]["achieved"] / ceil["hbm_read_GBps"], 4)
        dec["graph"] = {"ms_per_step": round(g_wall * 1e3, 4),
                        "weight_GBps_layer": round(r["wbytes"] / g_wall / 1e9, 1)}
        if "value" not in result:
            result.update({"value": dec["weight_GBps_layer"], "unit": "GB/s", "ms_per_step": dec["ms_per_step"],
                           "dtype": "mxfp8 x mxfp4 (e4m3 x e2m1, fp32 accumulate)",
                           "config": {"workload": name}, "roofline": dec["roofline"]})
        result["decode"] = dec
        del r["layer"], r["sets"], u["layer"], u["sets"]
        torch.cuda.empty_cache()
    if args.only in (None, "skewed"):
        name = "moe_prefill_t2048_zipf"
        r = bench_moe(name, args.steps, args.warmup, rotate=1)
        g_ms = r["stage_ms"]["grouped_gemm"]
        result["skewed"] = {"workload": name, "ms_per_step": round(r["ms"], 4),
                            "stages_ms": {k: round(v, 4) for k, v in r["stage_ms"].items()},
                            "touched_experts": r["touched"], "max_rows_per_expert": r["max_rows"],
                            "grouped_TFLOPs": round(r["flops"] / (g_ms * 1e-3) / 1e12, 1),
                            "touched_weight_GBps_grouped": round(r["wbytes"] / (g_ms * 1e-3) / 1e9, 1)}
        sk = result["skewed"]
        sk["frac_fp8_peak"] = round(sk["grouped_TFLOPs"] / PEAK_TFLOPS["e4m3"], 4)
        sk["traffic_grouped_gemm"] = measured_traffic(name)
        sk["frac_hbm_peak"] = round(sk["touched_weight_GBps_grouped"] / PEAK_HBM_GBS, 4)
        if ceil:
            sk["frac_of_measured_ceilings"] = {
                "mfma": round(sk["grouped_TFLOPs"] / ceil["mfma_e4m3xe2m1_random_TFLOPs"], 4),
                "hbm": round(sk["touched_weight_GBps_grouped"] / ceil["hbm_read_GBps"], 4)}
        del r["layer"], r["sets"]
        torch.cuda.empty_cache()
    if args.only in (None, "dense"):
        # the 16 x 32 x 4096 GEMM (203 KB: launch-bound, its time is what is reported)
        r0 = bench_dense(args.steps, args.warmup, name="dense_m16_n32_k4096")
        result["dense_small"] = {"workload": "dense_m16_n32_k4096", "us": round(r0["ms"] * 1e3, 2),
                                 "graph_us": round(r0["graph_ms"] * 1e3, 2)}
        r = bench_dense(args.steps, args.warmup)
        result["dense"] = {"workload": "dense_m64_n4096_k7168", "ms": round(r["ms"], 5),
                           "weight_GBps": round(r["gbs"], 1), "frac_hbm": round(r["gbs"] / PEAK_HBM_GBS, 4),
                           "TFLOPs": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
                           "graph": {"ms": round(r["graph_ms"], 5),
                                     "weight_GBps": round(r["wbytes"] / (r["graph_ms"] * 1e-3) / 1e9, 1)}}
    if args.only in (None, "variants"):
        result["fp4_variants"] = bench_fp4_variants(args.steps, args.warmup)
    if not args.no_cpu and args.only in (None, "prefill"):
        log("[bench] timing the CPU oracle on a bounded sample ...")
        result["cpu_baseline"] = cpu_baseline("moe_prefill_t16384_fp4")
        result["cpu_baseline"]["cpu_model"] = cpu_model()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
