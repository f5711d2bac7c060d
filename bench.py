#!/usr/bin/env python3
"""Benchmark of the block-scaled o_proj layer on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20]

Headline workload (one "step"): the A4W4 attention output projection at decode
size - X [64, 8192] BF16 ~ N(0,1) is quantized dynamically to MXFP4
(mx_quant_act_bf16) and multiplied with the pre-quantized MXFP4 weight
[7168, 8192] + E8M0 scales [7168, 256] (mx_gemm_a4w4_bf16) into BF16 Y
[64, 7168] (shapes: "Kimi-K3 DSpark O-Proj-only MXFP4", section "Exact
quantization coverage"; M = 8 concurrent requests x 8 draft positions).  Every
step reads a different copy of the weight (and activations) from a rotation
large enough to defeat the 256 MB Infinity Cache, so weights stream from HBM.
Steps are replayed from a HIP graph.  The printed JSON line also carries:
  roofline      the GEMM kernel's achieved HBM bandwidth (algorithmic bytes per
                launch / average launch time, HIP events on the launch stream)
  cpu_baseline  the CPU oracle timed on the same layer on the host cores
  also          the prefill layer (M = 8192), the PTPC FP8 A8W8 layers, the
                M sweep, the quantizer kernels, the offline weight
                conversions and the grouped MoE GEMM, each with its roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP4_TFLOPS = 10100.0   # dense MXFP4 / FP6 MFMA
PEAK_FP8_TFLOPS = 5000.0    # dense FP8 MFMA
PEAK_FP16_TFLOPS = 2500.0   # dense FP16 / BF16 MFMA
METRIC = "A4W4 o_proj GEMM TFLOP/s and GB/s (% roofline) at M=64 and M=8192, 1 GPU"
ROTATE_MIN_BYTES = 512 << 20


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--kernel-reps", type=int, default=30, help="graph replays per kernel-timing measurement")
    ap.add_argument("--no-extra", action="store_true", help="headline only (skip prefill / A8W8 / sweep)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarize two rocprofv3 --pmc runs of --profile-pass (FETCH_SIZE, then WRITE_SIZE) "
                         "into profiles/pmc_traffic.json and exit (no GPU needed)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="run each measured kernel a few times plus a plain copy of known size, for rocprofv3 --pmc")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------- helpers
def algorithmic_bytes(kind, M, N, K):
    if kind == "a4w4":
        return M * K // 2 + M * K // 32 + N * K // 2 + N * K // 32 + 2 * M * N
    if kind == "a8w8":
        return M * K + 4 * M + N * K + 4 * N + 2 * M * N
    if kind == "mxq":
        return 2 * M * K + M * K // 2 + M * K // 32
    if kind == "ptpcq":
        return 2 * M * K + M * K + 4 * M
    if kind == "mxw":  # offline weight conversion, FP32 in
        return 4 * M * K + M * K // 2 + M * K // 32
    if kind == "ptpcw":
        return 4 * M * K + M * K + 4 * M
    raise ValueError(kind)


class Ctx:
    def __init__(self):
        import torch
        from block_scaled_precision_act_amd import mxgemm
        if not os.path.exists(mxgemm.LIB_PATH):
            from block_scaled_precision_act_amd import build
            build.build()
        self.torch = torch
        self.mx = mxgemm
        mxgemm.lib()
        if not torch.cuda.is_available():
            raise RuntimeError("bench.py needs a GPU")
        self.dev = torch.device("cuda:0")
        self.weights = {}

    def weight(self, cfg_name, kind):
        """Quantized weight of a config (generated on the host, converted on the GPU), cached."""
        key = (cfg_name, kind)
        if key not in self.weights:
            from block_scaled_precision_act_amd import synth
            w = self.torch.from_numpy(synth.make_weight(synth.CONFIGS[cfg_name])).to(self.dev)
            self.weights[key] = self.mx.quant_weight_mx(w) if kind == "a4w4" else self.mx.quant_weight_ptpc(w)
            del w
        return self.weights[key]

    def stream(self):
        return self.torch.cuda.current_stream().cuda_stream

    def capture(self, thunks):
        torch = self.torch
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in thunks:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in thunks:
                f()
        torch.cuda.synchronize()
        return g

    def event_ms(self, g, reps):
        """Average ms per replay of graph g, HIP events on the replay stream."""
        torch = self.torch
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps


def ok(status, what):
    if status != 0:
        from block_scaled_precision_act_amd import mxgemm
        raise RuntimeError("%s failed: %s" % (what, mxgemm.status_string(status)))


def dev_bf16(ctx, bits):
    import numpy as np
    return ctx.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(ctx.torch.bfloat16).to(ctx.dev)


def rotation_count(bytes_per_set, cap=64):
    return max(2, min(cap, -(-ROTATE_MIN_BYTES // max(1, bytes_per_set))))


# ----------------------------------------------------------------------------- A4W4 layer
class A4W4Layer:
    """R rotating copies of (X, quantized W, outputs) for one shape."""

    def __init__(self, ctx, x_bits, qw, sw, rotate):
        torch, mx = ctx.torch, ctx.mx
        self.ctx = ctx
        self.M, self.K = x_bits.shape
        self.N = qw.shape[0]
        x0 = dev_bf16(ctx, x_bits)
        self.R = rotate
        self.x = [x0] + [x0.clone() for _ in range(rotate - 1)]
        self.qw = [qw] + [qw.clone() for _ in range(rotate - 1)]
        self.sw = [sw] + [sw.clone() for _ in range(rotate - 1)]
        M, N, K = self.M, self.N, self.K
        self.qa = [torch.empty((M, K // 2), dtype=torch.uint8, device=ctx.dev) for _ in range(rotate)]
        self.sa = [torch.empty((M, K // 32), dtype=torch.uint8, device=ctx.dev) for _ in range(rotate)]
        self.y = [torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev) for _ in range(rotate)]
        self.ws = mx.mx_gemm_a4w4_workspace_bytes(M, N, K)  # shared by the steps (they run in stream order)
        # zero-filled once; every call leaves its counters at zero again
        self.wbuf = torch.zeros(max(self.ws, 16), dtype=torch.uint8, device=ctx.dev)

    def quant(self, r):
        mx, ctx = self.ctx.mx, self.ctx
        return lambda: ok(mx.mx_quant_act_bf16(self.x[r].data_ptr(), self.M, self.K, self.qa[r].data_ptr(),
                                               self.sa[r].data_ptr(), ctx.stream()), "mx_quant_act_bf16")

    def gemm(self, r):
        mx, ctx = self.ctx.mx, self.ctx
        return lambda: ok(mx.mx_gemm_a4w4_bf16(self.qa[r].data_ptr(), self.sa[r].data_ptr(), self.qw[r].data_ptr(),
                                               self.sw[r].data_ptr(), self.y[r].data_ptr(), self.M, self.N, self.K,
                                               self.wbuf.data_ptr(), self.ws, ctx.stream()), "mx_gemm_a4w4_bf16")

    def step(self, r):
        q, g = self.quant(r), self.gemm(r)
        return lambda: (q(), g())

    def fused(self, r):
        """The same layer through the one-call entry (BF16 X in, BF16 Y out)."""
        mx, ctx = self.ctx.mx, self.ctx
        if not hasattr(self, "lws"):
            self.lws = mx.mx_linear_a4w4_workspace_bytes(self.M, self.N, self.K)
            self.lbuf = ctx.torch.zeros(max(self.lws, 256), dtype=ctx.torch.uint8, device=ctx.dev)
        return lambda: ok(mx.mx_linear_a4w4_bf16(self.x[r].data_ptr(), self.qw[r].data_ptr(), self.sw[r].data_ptr(),
                                                 self.y[r].data_ptr(), self.M, self.N, self.K, self.lbuf.data_ptr(),
                                                 self.lws, ctx.stream()), "mx_linear_a4w4_bf16")


class A8W8Layer:
    def __init__(self, ctx, x_bits, qw, sw, rotate):
        torch = ctx.torch
        self.ctx = ctx
        self.M, self.K = x_bits.shape
        self.N = qw.shape[0]
        x0 = dev_bf16(ctx, x_bits)
        self.R = rotate
        self.x = [x0] + [x0.clone() for _ in range(rotate - 1)]
        self.qw = [qw] + [qw.clone() for _ in range(rotate - 1)]
        self.sw = [sw] + [sw.clone() for _ in range(rotate - 1)]
        M, N, K = self.M, self.N, self.K
        self.qa = [torch.empty((M, K), dtype=torch.uint8, device=ctx.dev) for _ in range(rotate)]
        self.sa = [torch.empty((M,), dtype=torch.float32, device=ctx.dev) for _ in range(rotate)]
        self.y = [torch.empty((M, N), dtype=torch.bfloat16, device=ctx.dev) for _ in range(rotate)]
        # split-K workspace (decode sizes): allocated and zeroed once, outside the timed region
        self.ws = ctx.mx.gemm_a8w8_ptpc_workspace_bytes(M, N, K)
        self.wbuf = torch.zeros(max(self.ws, 256), dtype=torch.uint8, device=ctx.dev)

    def quant(self, r):
        mx, ctx = self.ctx.mx, self.ctx
        return lambda: ok(mx.ptpc_quant_act_fp8(self.x[r].data_ptr(), self.M, self.K, self.qa[r].data_ptr(),
                                                self.sa[r].data_ptr(), ctx.stream()), "ptpc_quant_act_fp8")

    def gemm(self, r):
        mx, ctx = self.ctx.mx, self.ctx
        return lambda: ok(mx.gemm_a8w8_ptpc_bf16(self.qa[r].data_ptr(), self.sa[r].data_ptr(), self.qw[r].data_ptr(),
                                                 self.sw[r].data_ptr(), self.y[r].data_ptr(), self.M, self.N, self.K,
                                                 self.wbuf.data_ptr(), self.ws, ctx.stream()), "gemm_a8w8_ptpc_bf16")

    def step(self, r):
        q, g = self.quant(r), self.gemm(r)
        return lambda: (q(), g())


# Graph replays leave the GPU idle for several us between one replay's last kernel and the next one's first;
# kernel timings capture at least this many launches per graph, so that gap is spread thin.
LAUNCHES_PER_GRAPH = 160


def cycled_graph(ctx, thunks):
    """A graph cycling over the calls `thunks` (e.g. one per rotated copy) at least LAUNCHES_PER_GRAPH times
    in all, and its call count."""
    m = max(1, -(-LAUNCHES_PER_GRAPH // len(thunks)))
    return ctx.capture(list(thunks) * m), m * len(thunks)


def graph_ms(ctx, thunks, reps):
    """Average ms per call over about reps x len(thunks) calls (at least two graph replays)."""
    g, n = cycled_graph(ctx, thunks)
    return ctx.event_ms(g, max(2, -(-reps * len(thunks) // n))) / n


def kernel_ms(ctx, layer, which, reps):
    return graph_ms(ctx, [getattr(layer, which)(r) for r in range(layer.R)], reps)


SUSTAIN_S = 0.05
STEPS_PER_GRAPH = 1000


def sustained_entry(ctx, layer, which, reps, kind):
    """The same kernel timing after SUSTAIN_S seconds of back-to-back replays of the same graph: the clocks
    the kernel settles at under sustained use.  Starting from lighter work, the M = 8192 GEMM runs its first
    ~50 launches ~15% slower than later ones, while the decode GEMM gets a few % slower under sustained
    load; both figures are reported, the primary ones keep the short warm-up."""
    import time
    torch = ctx.torch
    g, n = cycled_graph(ctx, [getattr(layer, which)(r) for r in range(layer.R)])
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SUSTAIN_S:
        g.replay()
        torch.cuda.synchronize()
    ms = ctx.event_ms(g, max(2, -(-reps * layer.R // n))) / n
    r = roofline_gemm(kind, layer.M, layer.N, layer.K, ms)
    return {"warmup_s": SUSTAIN_S, "kernel_us": r["kernel_us"], "achieved": r["achieved"], "unit": r["unit"],
            "frac": r["frac"]}


def roofline_gemm(kind, M, N, K, ms):
    flop = 2.0 * M * N * K
    byt = algorithmic_bytes(kind, M, N, K)
    tflops = flop / (ms * 1e-3) / 1e12
    gbs = byt / (ms * 1e-3) / 1e9
    peak_c = PEAK_FP4_TFLOPS if kind == "a4w4" else PEAK_FP8_TFLOPS
    t_hbm = byt / (PEAK_HBM_GBS * 1e9)
    t_mfma = flop / (peak_c * 1e12)
    if t_hbm >= t_mfma:
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None, "kernel_us": round(ms * 1e3, 3),
                "tflops": round(tflops, 2), "alg_bytes_per_launch": byt}
    return {"bound": "mfma", "achieved": round(tflops, 1), "peak": peak_c, "unit": "TFLOP/s",
            "frac": round(tflops / peak_c, 4), "traffic": None, "kernel_us": round(ms * 1e3, 3),
            "gbs": round(gbs, 1), "alg_flop_per_launch": flop}


def roofline_quant(kind, M, K, ms):
    byt = algorithmic_bytes(kind, M, 0, K)
    gbs = byt / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel_us": round(ms * 1e3, 3), "alg_bytes_per_launch": byt}


def pmc_traffic(kernel_key):
    """HBM traffic per launch from the committed rocprofv3 --pmc summary, if it
    was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("kernels", {}).get(kernel_key)


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_precision_act_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------------------- workloads
def make_a4w4(ctx, cfg_name, M=None, rotate=None):
    from block_scaled_precision_act_amd import synth
    cfg = synth.CONFIGS[cfg_name]
    x_bits = synth.make_activations(cfg, M)
    qw, sw = ctx.weight(cfg_name, "a4w4")  # offline weight conversion, on the GPU
    Mx, K = x_bits.shape
    per_set = algorithmic_bytes("a4w4", Mx, cfg["N"], K) + 2 * Mx * K
    R = rotate or rotation_count(per_set)
    return A4W4Layer(ctx, x_bits, qw, sw, R)


def make_a8w8(ctx, cfg_name, rotate=None, M=None):
    from block_scaled_precision_act_amd import synth
    cfg = synth.CONFIGS[cfg_name]
    x_bits = synth.make_activations(cfg, M)
    qw, sw = ctx.weight(cfg_name, "a8w8")
    Mx, K = x_bits.shape
    per_set = algorithmic_bytes("a8w8", Mx, cfg["N"], K) + 2 * Mx * K
    R = rotate or rotation_count(per_set)
    return A8W8Layer(ctx, x_bits, qw, sw, R)


def time_steps(ctx, layer, steps, warmup):
    """Wall-clock time of exactly `steps` layer steps (step i on rotated copy i mod R), captured as graphs of
    up to STEPS_PER_GRAPH consecutive steps and replayed back to back.  A graph launch costs the host 15-30 us
    before its first kernel starts, and the next launch can wait on it, so the timed steps go in as few
    launches as possible: one for up to STEPS_PER_GRAPH steps.  Warm-up: ceil(warmup / R) replays of all R copies,
    then one untimed replay of each timed graph (its first launch)."""
    torch = ctx.torch
    R = layer.R
    cache = {}
    timed = []
    for s0 in range(0, steps, STEPS_PER_GRAPH):
        key = (s0 % R, min(STEPS_PER_GRAPH, steps - s0))
        if key not in cache:
            cache[key] = ctx.capture([layer.step((key[0] + i) % R) for i in range(key[1])])
        timed.append(cache[key])
    full = ctx.capture([layer.step(r) for r in range(R)])
    for _ in range(-(-warmup // R)):
        full.replay()
    for g in cache.values():
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in timed:
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def layer_entry(ctx, layer, kind, args, label):
    M, N, K = layer.M, layer.N, layer.K
    gemm_ms = kernel_ms(ctx, layer, "gemm", args.kernel_reps)
    quant_ms = kernel_ms(ctx, layer, "quant", args.kernel_reps)
    step_ms = time_steps(ctx, layer, max(layer.R, 40), 10)
    e = {"workload": label, "M": M, "N": N, "K": K, "rotation": layer.R,
         "layer_ms": round(step_ms, 5), "layer_tflops": round(2.0 * M * N * K / (step_ms * 1e-3) / 1e12, 2),
         "gemm": roofline_gemm(kind, M, N, K, gemm_ms),
         "quant": roofline_quant("mxq" if kind == "a4w4" else "ptpcq", M, K, quant_ms)}
    if kind == "a8w8":
        e["gemm"]["note"] = ("E4M3 operands widened exactly to FP16 and run on FP16 MFMA (peak %.0f TFLOP/s); "
                             "frac is against the FP8 peak" % PEAK_FP16_TFLOPS)
    return e


def one_call_layer_entry(ctx, args):
    """The one-call A4W4 layer (mx_linear_a4w4_bf16: one kernel for M <= 8, quantizing X inside the split-K
    GEMM's workgroups; the quantizer and the GEMM above that) beside the two-launch layer (quantizer + GEMM
    entries), o_proj weight, M = 1, 8, 16, 64."""
    out = {}
    for Ms in (1, 8, 16, 64):
        lay = make_a4w4(ctx, "oproj_decode_a4w4", M=Ms)
        # alternated, best of two each: the first of a run of timings can catch the clocks still rising
        one_ms, two_ms = float("inf"), float("inf")
        for _ in range(2):
            one_ms = min(one_ms, kernel_ms(ctx, lay, "fused", args.kernel_reps))
            two_ms = min(two_ms, kernel_ms(ctx, lay, "step", args.kernel_reps))
        # algorithmic bytes of the layer: BF16 X in, the MXFP4 weight and its scales in, BF16 Y out
        byt = 2 * Ms * lay.K + lay.N * lay.K // 2 + lay.N * lay.K // 32 + 2 * Ms * lay.N
        gbs = byt / (one_ms * 1e-3) / 1e9
        out["M=%d" % Ms] = {"one_call_us": round(one_ms * 1e3, 3), "two_launch_us": round(two_ms * 1e3, 3),
                            "one_call_path": "one launch" if Ms <= 8 else "quantizer + GEMM",
                            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "alg_bytes_per_launch": byt}
        del lay
        ctx.torch.cuda.empty_cache()
    return {"workload": "A4W4 o_proj layer BF16 X [M, 8192] -> BF16 Y [M, 7168], W [7168, 8192] MXFP4; "
                        "one call (one launch with the quantization inside the split-K GEMM for M <= 8) vs "
                        "quantizer + GEMM entries, graph-replayed, rotated copies", "by_M": out}


def weight_conversion_entry(ctx, args):
    """The offline weight conversions (FP32 -> MXFP4 + E8M0, FP32 -> E4M3 + FP32 channel scale) on the
    o_proj weight [7168, 8192], two rotated copies, graph-replayed."""
    torch, mx = ctx.torch, ctx.mx
    from block_scaled_precision_act_amd import synth
    cfg = synth.CONFIGS["oproj_decode_a4w4"]
    N, K = cfg["N"], cfg["K"]
    w0 = torch.from_numpy(synth.make_weight(cfg)).to(ctx.dev)
    ws = [w0, w0.flip(0).contiguous()]
    u8 = torch.uint8
    q4 = [torch.empty((N, K // 2), dtype=u8, device=ctx.dev) for _ in ws]
    s4 = [torch.empty((N, K // 32), dtype=u8, device=ctx.dev) for _ in ws]
    q8 = [torch.empty((N, K), dtype=u8, device=ctx.dev) for _ in ws]
    s8 = [torch.empty((N,), dtype=torch.float32, device=ctx.dev) for _ in ws]
    out = {"workload": "offline weight conversion of W [%d, %d] FP32" % (N, K), "rotation": len(ws)}
    for key, kind, fn, qs, ss in (("mxfp4", "mxw", mx.mx_quant_weight_f32, q4, s4),
                                  ("ptpc_fp8", "ptpcw", mx.ptpc_quant_weight_f32, q8, s8)):
        thunks = [(lambda i=i: ok(fn(ws[i].data_ptr(), N, K, qs[i].data_ptr(), ss[i].data_ptr(), ctx.stream()),
                                  key)) for i in range(len(ws))]
        ms = graph_ms(ctx, thunks, args.kernel_reps)
        byt = algorithmic_bytes(kind, N, 0, K)
        gbs = byt / (ms * 1e-3) / 1e9
        out[key] = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel_us": round(ms * 1e3, 3),
                    "alg_bytes_per_launch": byt}
    del ws, w0, q4, s4, q8, s8
    torch.cuda.empty_cache()
    return out


def grouped_entry(ctx, args, name="moe_grouped_a4w4"):
    """Grouped A4W4 GEMM over MoE experts (synthetic shapes: 64 tokens x top-8 over 32 experts of
    [7168, 2048], the down projections; or of [2048, 7168], the up projections), two rotated sets of
    expert weights, graph-replayed."""
    import numpy as np
    torch, mx = ctx.torch, ctx.mx
    from block_scaled_precision_act_amd import synth
    cfg = synth.CONFIGS[name]
    G, N, K = cfg["G"], cfg["N"], cfg["K"]
    counts = synth.route_counts(cfg["route"], cfg["tokens"], cfg["topk"], G)
    T, max_rows = int(counts.sum()), int(counts.max())
    offsets = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32, device=ctx.dev)
    x = torch.from_numpy(synth.make_activations(cfg, T).view(np.int16)).view(torch.bfloat16).to(ctx.dev)
    qa, sa = mx.quant_act_mx(x)
    qw1, sw1 = mx.quant_weight_mx(torch.from_numpy(synth.make_weight(cfg)).to(ctx.dev))
    # distinct experts as row rotations of one MXFP4 draw (every expert a valid [N, K] weight)
    R = 2
    qws = [torch.stack([torch.roll(qw1, (37 * e + 11 * r) % N, 0) for e in range(G)]) for r in range(R)]
    sws = [torch.stack([torch.roll(sw1, (37 * e + 11 * r) % N, 0) for e in range(G)]) for r in range(R)]
    y = torch.empty((T, N), dtype=torch.bfloat16, device=ctx.dev)
    thunks = [(lambda r=r: ok(mx.mx_gemm_a4w4_grouped_bf16(qa.data_ptr(), sa.data_ptr(), qws[r].data_ptr(),
                                                           sws[r].data_ptr(), y.data_ptr(), offsets.data_ptr(), G,
                                                           max_rows, N, K, ctx.stream()), "grouped"))
              for r in range(R)]
    ms = graph_ms(ctx, thunks, args.kernel_reps)
    used = counts > 0
    byt = int(used.sum()) * (N * K // 2 + N * K // 32) + T * (K // 2 + K // 32) + 2 * T * N
    gbs = byt / (ms * 1e-3) / 1e9
    out = {"workload": "grouped MoE A4W4: %d tokens x top-%d over %d experts of [%d, %d], rows per expert %d..%d"
                       % (cfg["tokens"], cfg["topk"], G, N, K, int(counts.min()), max_rows),
           "rotation": R, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(gbs / PEAK_HBM_GBS, 4), "kernel_us": round(ms * 1e3, 3), "alg_bytes_per_launch": byt,
           "tflops": round(2.0 * T * N * K / (ms * 1e-3) / 1e12, 2)}
    del qws, sws, qw1, sw1, x, qa, sa, y
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- CPU baseline
def host_threads():
    """(threads the oracle uses, CPUs this process may run on): all of them unless OMP_NUM_THREADS
    sets a smaller share of the host."""
    import oracle
    cpus = oracle.default_threads()
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return (min(cpus, share) if share > 0 else cpus), cpus


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _timed(fn, budget_s, max_reps=200):
    t0 = time.perf_counter()
    reps = 0
    while True:
        fn()
        reps += 1
        if time.perf_counter() - t0 > budget_s or reps >= max_reps:
            break
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline():
    """The oracle (plain C, exact arithmetic, row-parallel) on the host: the headline decode layer in
    full for about 10 s, then every configuration of the layer for about 2 s each, large ones on a
    sample of rows (MXFP4 / PTPC quantization of those rows + their exact GEMM against all of W),
    with the full-layer time extrapolated from the rows per second."""
    import oracle
    from block_scaled_precision_act_amd import synth
    threads, cpus = host_threads()
    cfg = synth.CONFIGS["oproj_decode_a4w4"]
    x_bits = synth.make_activations(cfg)
    qw, sw = oracle.mx_quant_f32(synth.make_weight(cfg), nthreads=threads)  # offline, not timed
    M, N, K = cfg["M"], cfg["N"], cfg["K"]

    def layer():
        qa, sa = oracle.mx_quant_bf16(x_bits, nthreads=threads)
        oracle.gemm_a4w4_at(qa, sa, qw, sw, nthreads=threads)

    sec, reps = _timed(layer, 10.0)
    out = {"value": round(2.0 * M * N * K / sec / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
           "host_cpus": cpus, "cpu_model": cpu_model(), "kind": "oracle",
           "sample": "full o_proj decode layer (MXFP4 quantization of X [64, 8192] + exact A4W4 GEMM against "
                     "W [7168, 8192]), %d repetition(s), %.2f s each" % (reps, sec)}
    per = {}
    weights = {}
    for name, rows in (("tiny_a4w4", None), ("oproj_decode_a4w4", None), ("oproj_prefill_a4w4", 64),
                       ("msweep_outlier_a4w4", 64), ("ptpc_a8w8_m64", None), ("ptpc_a8w8_m8192", 64)):
        c = synth.CONFIGS[name]
        Mc, Nc, Kc = c["M"], c["N"], c["K"]
        Ms = Mc if rows is None else rows
        x = synth.make_activations(c, Ms)
        key = (c["w"], c["kind"], Nc, Kc)
        if key not in weights:
            w = synth.make_weight(c)
            weights[key] = (oracle.mx_quant_f32 if c["kind"] == "a4w4" else oracle.ptpc_quant_f32)(w, nthreads=threads)
        wq, ws_ = weights[key]
        if c["kind"] == "a4w4":
            def run():
                qa, sa = oracle.mx_quant_bf16(x, nthreads=threads)
                oracle.gemm_a4w4_at(qa, sa, wq, ws_, nthreads=threads)
        else:
            def run():
                qa, sa = oracle.ptpc_quant_bf16(x, nthreads=threads)
                oracle.gemm_a8w8_at(qa, sa, wq, ws_, nthreads=threads)
        s_, r_ = _timed(run, 2.0)
        full_s = s_ * Mc / Ms
        per[name] = {"M": Mc, "N": Nc, "K": Kc, "rows_timed": Ms, "reps": r_, "sample_s": round(s_, 4),
                     "full_layer_s": round(full_s, 3), "tflops": round(2.0 * Mc * Nc * Kc / full_s / 1e12, 6)}
    out["per_config"] = per
    return out


# ----------------------------------------------------------------------------- profile pass
def profile_pass(ctx):
    """Each measured kernel a few times + a plain device copy of known size,
    for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs."""
    torch = ctx.torch
    src = torch.empty(256 << 20, dtype=torch.uint8, device=ctx.dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    dec = make_a4w4(ctx, "oproj_decode_a4w4")
    for r in range(min(4, dec.R)):
        dec.quant(r)()
        dec.gemm(r)()
    torch.cuda.synchronize()
    one = make_a4w4(ctx, "oproj_decode_a4w4", M=1)
    for r in range(min(4, one.R)):
        one.fused(r)()
    torch.cuda.synchronize()
    pre = make_a4w4(ctx, "oproj_prefill_a4w4", rotate=2)
    for r in range(2):
        pre.quant(r)()
        pre.gemm(r)()
    torch.cuda.synchronize()
    log("profile pass done (copy of %d bytes x3)" % src.numel())


# ----------------------------------------------------------------------------- PMC summary
# Kernels whose HBM traffic the bench reports: key -> (name fragment, grid size in threads or None)
PMC_KERNELS = {
    "gemm_splitk_fp4_m64": ("gemm_splitk_fp4<2, 4, 8, 4, false>", None),
    "gemm_tile224_fp4_m8192": ("gemm_tile224_fp4<true>", 1024 * 256),
    "linear_splitk_fused_m1": ("gemm_splitk_fp4<1, 5, 8, 4, true>", None),
}
COPY_BYTES = 256 << 20  # the profile pass copies 256 MiB device -> device


def read_pmc(folder, counter):
    """Per-dispatch values (KiB) of one counter from rocprofv3 --output-format csv files."""
    import csv
    rows = []
    for dirpath, _, files in os.walk(folder):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(dirpath, fn), newline="") as f:
                    for r in csv.DictReader(f):
                        if r["Counter_Name"] == counter:
                            rows.append((r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])))
    if not rows:
        raise SystemExit("no %s rows under %s" % (counter, folder))
    return rows


def pmc_summary(fetch_dir, write_dir):
    fetch, write = read_pmc(fetch_dir, "FETCH_SIZE"), read_pmc(write_dir, "WRITE_SIZE")

    def mean_of(rows, frag, grid):
        v = [val for name, g, val in rows if frag in name and (grid is None or g == grid)]
        return (sum(v) / len(v), len(v)) if v else (None, 0)

    # the copy: the largest FETCH among kernels whose name says copy; its writes likewise
    cf = max((val for name, _, val in fetch if "opy" in name), default=None)
    cw = max((val for name, _, val in write if "opy" in name), default=None)
    if not cf or not cw:
        raise SystemExit("copy dispatch not found in the PMC runs")
    f_fetch, f_write = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    out = {"source_hash": source_hash(),
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cf, "write_kib": cw,
                                "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4)},
           "kernels": {}, "detail": {}}
    for key, (frag, grid) in PMC_KERNELS.items():
        mf, nf = mean_of(fetch, frag, grid)
        mw, nw = mean_of(write, frag, grid)
        if mf is None or mw is None:
            continue
        b = mf * 1024.0 * f_fetch + mw * 1024.0 * f_write
        out["kernels"][key] = int(round(b))
        out["detail"][key] = {"fetch_kib": round(mf, 1), "write_kib": round(mw, 1), "dispatches": [nf, nw],
                              "fetch_bytes": int(round(mf * 1024.0 * f_fetch)),
                              "write_bytes": int(round(mw * 1024.0 * f_write))}
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out, indent=1))


# ----------------------------------------------------------------------------- main
def main():
    args = parse_args()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the layer on one GPU only: the library has no multi-GPU path "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.steps <= 0 or args.warmup < 0:
        print("--steps must be > 0 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    ctx = Ctx()
    torch = ctx.torch
    if args.profile_pass:
        profile_pass(ctx)
        return

    log("generating the decode workload (X [64, 8192], W [7168, 8192])")
    dec = make_a4w4(ctx, "oproj_decode_a4w4")
    log("rotation: %d weight/activation copies" % dec.R)
    gemm_ms = kernel_ms(ctx, dec, "gemm", args.kernel_reps)
    quant_ms = kernel_ms(ctx, dec, "quant", args.kernel_reps)
    log("decode GEMM %.2f us, quant %.2f us" % (gemm_ms * 1e3, quant_ms * 1e3))

    ms_per_step = time_steps(ctx, dec, args.steps, args.warmup)
    M, N, K = dec.M, dec.N, dec.K
    value = 2.0 * M * N * K / (ms_per_step * 1e-3) / 1e12
    log("step %.3f us -> %.2f TFLOP/s" % (ms_per_step * 1e3, value))

    roof = roofline_gemm("a4w4", M, N, K, gemm_ms)
    roof["traffic"] = pmc_traffic("gemm_splitk_fp4_m64")
    roof["kernel"] = "gemm_splitk_fp4<2, 4, 8, 4, false>"
    sustained = sustained_entry(ctx, dec, "gemm", args.kernel_reps, "a4w4")
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "mxfp4 (e2m1 x e2m1, e8m0 scales, fp32 accumulate, bf16 out)",
        "data": "synthetic (seeded SplitMix64; X ~ N(0,1) bf16, W ~ N(0,0.01) fp32 quantized on the GPU)",
        "config": {"workload": "A4W4 o_proj decode layer: BF16 X [64, 8192] -> dynamic MXFP4 -> A4W4 GEMM vs "
                               "MXFP4 W [7168, 8192] + E8M0 [7168, 256] -> BF16 Y [64, 7168]",
                   "M": M, "N": N, "K": K, "rotation": dec.R, "graph_replay": True},
        "roofline": roof,
        "layer_breakdown_us": {"quant": round(quant_ms * 1e3, 3), "gemm": round(gemm_ms * 1e3, 3)},
        "gemm_sustained": sustained,
    }
    del dec
    torch.cuda.empty_cache()

    if not args.no_extra:
        also = {}
        log("prefill A4W4 (M = 8192)")
        pre = make_a4w4(ctx, "oproj_prefill_a4w4", rotate=2)
        also["a4w4_prefill_m8192"] = layer_entry(ctx, pre, "a4w4", args, "oproj_prefill_a4w4")
        also["a4w4_prefill_m8192"]["gemm"]["traffic"] = pmc_traffic("gemm_tile224_fp4_m8192")
        also["a4w4_prefill_m8192"]["gemm"]["kernel"] = "gemm_tile224_fp4<true>"
        also["a4w4_prefill_m8192"]["gemm_sustained"] = sustained_entry(ctx, pre, "gemm", args.kernel_reps, "a4w4")
        del pre
        ctx.weights.clear()
        torch.cuda.empty_cache()
        sweep = {}
        for Ms in (1, 16, 128, 512, 2048):
            log("outlier sweep M = %d" % Ms)
            lay = make_a4w4(ctx, "msweep_outlier_a4w4", M=Ms)
            sweep["M=%d" % Ms] = layer_entry(ctx, lay, "a4w4", args, "msweep_outlier_a4w4")
            del lay
            torch.cuda.empty_cache()
        also["a4w4_msweep_outliers"] = sweep
        ctx.weights.clear()
        for name in ("ptpc_a8w8_m64", "ptpc_a8w8_m8192"):
            log("A8W8 %s" % name)
            lay = make_a8w8(ctx, name, rotate=2 if name.endswith("8192") else None)
            also[name] = layer_entry(ctx, lay, "a8w8", args, name)
            del lay
            torch.cuda.empty_cache()
        log("mid-size M")
        mid = {}
        for kind, cfg_name in (("a4w4", "oproj_prefill_a4w4"), ("a8w8", "ptpc_a8w8_m8192")):
            for Ms in (256, 512):
                lay = (make_a4w4(ctx, cfg_name, M=Ms) if kind == "a4w4" else make_a8w8(ctx, cfg_name, M=Ms))
                mid["%s M=%d" % (kind, Ms)] = layer_entry(ctx, lay, kind, args, "%s rows 0 .. %d" % (cfg_name, Ms - 1))
                del lay
                torch.cuda.empty_cache()
            ctx.weights.clear()
        also["mid_m"] = {"workload": "o_proj layer (N = 7168, K = 8192) at M = 256 and 512, the first M rows of the "
                                     "M = 8192 activations: the 128-row tiles with copy and MFMA waves (two K parts "
                                     "at M = 256)", "by_case": mid}
        log("one-call layer")
        also["a4w4_one_call_layer"] = one_call_layer_entry(ctx, args)
        log("offline weight conversion")
        also["weight_conversion"] = weight_conversion_entry(ctx, args)
        log("grouped MoE A4W4")
        also["moe_grouped_a4w4"] = grouped_entry(ctx, args)
        also["moe_grouped_up_a4w4"] = grouped_entry(ctx, args, "moe_grouped_up_a4w4")
        out["also"] = also

    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline()
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
