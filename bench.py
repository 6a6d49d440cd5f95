"""Benchmark of the H-BitLinear forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Default workload: the 3B-like layer chain at 8192 tokens, all INT4 activations
(plain BitLinear QKV 4096 -> 12288 and gate/up 4096 -> 32768, H-BitLinear Wo
4096 -> 4096 and Wdown 16384 -> 4096), bf16 in and out.  A step is one pass of
the hot path over one batch: the forward of the four layers (norm, Hadamard
where the layer has it, per-token INT4 quantisation, the integer product on the
FP6 x FP4 matrix cores, the rescale) against weights that were ternarised and
converted to FP4 once beforehand, as a deployment holds them.  The weight
ternarisation and conversion are timed separately.  Inputs are seeded
synthetic arrays already resident in HBM; exactly --steps steps are timed,
launched back to back with HIP events around every kernel (the same steps
replayed from a HIP graph are reported beside them).  The chain's four layers together hold
about 1.6 GB of inputs, weights, codes and outputs, far more than the 256 MB
last-level cache; the single-layer workloads rotate over enough distinct
buffer sets (> 512 MiB) that the cache cannot hold a step's inputs.

Prints one JSON line: tokens/s and TOPS of the step; for the kernel that takes
the most time per step, the algorithmic work per launch over its average
launch time (HIP events on the launch stream, recorded around each kernel of
the timed steps) against the MI355X peak and against ceilings measured in
the same process; the same figures for the other workloads (1.3B-like Wo with
INT8 codes, 7B-like Wdown, decode at 1, 16 and 64 tokens); and the CPU oracle
timed on a bounded row sample on the host cores.
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

METRIC = "H-BitLinear tokens/s + TOPS (a4/a8 × ternary W) and % of HBM/MFMA roofline"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_I8_TOPS = 5000.0          # MI355X dense INT8 MFMA, TOP/s
PEAK_F6F4_TOPS = 10100.0       # MI355X dense FP6 / FP4 MFMA, TFLOP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 576 << 20       # > 2 x 256 MB last-level cache
DECODE_W_BYTES = 8 << 20       # 2-bit weights of the 8192 x 4096 decode layer

_PEAKS = None


def log(msg):
    """Progress of the run on stderr (stdout carries only the JSON line)."""
    print("[bench] " + msg, file=sys.stderr, flush=True)


def cpu_model() -> str:
    """The host CPU as /proc/cpuinfo names it, with its family and model
    numbers (a virtualised host may report only a generic model name)."""
    fields = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" in line:
                    k, v = (x.strip() for x in line.split(":", 1))
                    if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                        fields[k] = v
                if not line.strip() and fields:
                    break  # the first processor's block is enough
    except OSError:
        pass
    name = fields.get("model name", "unknown")
    nums = ", ".join("%s %s" % (k, fields[k]) for k in ("cpu family", "model", "stepping") if k in fields)
    return "%s (%s)" % (name, nums) if nums else name


def measured_peaks():
    """Ceilings measured on this GPU by the probe kernels of libhbl_peaks.so
    (built beside libhbl.so), timed with HIP events on the stream they run on:
      * a 512 MiB streaming copy (read + write bytes), and a 32 MiB streaming
        write (the output burst of one wave of FP6 x FP4 GEMM tiles),
      * streaming reads of 8 MiB (the decode layer's 2-bit weights) and of
        64 MiB, each launch replayed from a HIP graph over buffers rotated
        past the last-level cache,
      * an empty 256-block kernel replayed from a graph (the launch floor),
      * loops of dense i8, FP6 x FP4 and bf16 matrix-core instructions on
        register operands,
      * the data path of one compute unit: LDS reads, LDS-direct loads, and
        both mixed with FP6 x FP4 instructions in the proportions of one K
        step of the FP6 x FP4 GEMM tile (with and without its barrier).
    Each figure is the best of 3 timed rounds after a warm-up.  Computed once."""
    global _PEAKS
    if _PEAKS is not None:
        return _PEAKS
    import ctypes

    import torch
    from bit_bitlinear_amd import build as hbl_build

    if not os.path.exists(hbl_build.PEAKS_LIB):
        raise RuntimeError("%s not found; build it with __graft_entry__.build()" % hbl_build.PEAKS_LIB)
    lib = ctypes.CDLL(hbl_build.PEAKS_LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.hbl_peak_copy.argtypes = [P, P, I64, P]
    lib.hbl_peak_read.argtypes = [P, I64, P, I64, P]
    lib.hbl_peak_read_sink_len.argtypes = [I64]
    lib.hbl_peak_read_sink_len.restype = I64
    lib.hbl_peak_empty.argtypes = [I32, P]
    lib.hbl_peak_mfma.argtypes = [I32, P, I64, I32, I32, P]
    lib.hbl_peak_mfma_ops.argtypes = [I32, I32, I32]
    lib.hbl_peak_mfma_ops.restype = I64
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def cur():
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def best_us(launch, reps=5):
        launch()
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                launch()
            e1.record(stream)
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            best = us if best is None else min(best, us)
        return best

    def graph_best_us(launches):
        """One graph holding every launch once; microseconds per launch."""
        for f in launches:
            f()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for f in launches:
                f()
        us = best_us(g.replay, reps=3) / len(launches)
        del g
        return us

    def ok(rc, what):
        if rc != 0:
            raise RuntimeError("%s failed (%d)" % (what, rc))

    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def copy():
        ok(lib.hbl_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, sp), "copy")

    out = {"hbm_copy_GBps": round(2 * nbytes / (best_us(copy) * 1e-6) / 1e9, 1)}
    # a 32 MiB streaming write (the output of one wave of 256 x 256 bf16 GEMM tiles on 256 compute units)
    # over distinct slices of the 512 MiB buffer, graph-replayed
    wsize = 32 << 20
    lib.hbl_peak_write.argtypes = [P, I64, P]
    wbase = dst.data_ptr()
    launches = [lambda i=i: ok(lib.hbl_peak_write(ctypes.c_void_p(wbase + i * wsize), wsize, cur()), "write")
                for i in range(nbytes // wsize)]
    us = graph_best_us(launches)
    out["hbm_write_32MiB_GBps"] = round(wsize / (us * 1e-6) / 1e9, 1)
    out["hbm_write_32MiB_us"] = round(us, 3)
    del dst
    # streaming reads at the decode layer's weight size and at 64 MiB, over
    # distinct slices of the 512 MiB buffer (every replay reads cold data)
    for size, key in ((DECODE_W_BYTES, "hbm_read_8MiB_GBps"), (64 << 20, "hbm_read_64MiB_GBps")):
        slices = nbytes // size
        sink = torch.empty(lib.hbl_peak_read_sink_len(size), dtype=torch.int32, device=dev)
        base = src.data_ptr()
        # the stream is read at call time: inside a graph capture it is the capture stream
        launches = [lambda i=i: ok(lib.hbl_peak_read(ctypes.c_void_p(base + i * size), size,
                                                    ctypes.c_void_p(sink.data_ptr()), sink.numel(), cur()), "read")
                    for i in range(slices)]
        us = graph_best_us(launches)
        out[key] = round(size / (us * 1e-6) / 1e9, 1)
        out[key.replace("GBps", "us")] = round(us, 3)
        del sink
    del src
    out["launch_floor_us"] = round(graph_best_us([lambda: ok(lib.hbl_peak_empty(256, cur()), "empty")] * 64), 3)
    blocks, iters = 2048, 2000
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    for kind, key in ((0, "mfma_i8_TOPS"), (1, "mfma_f6f4_TFLOPS"), (2, "mfma_bf16_TFLOPS")):
        def run(kind=kind):
            ok(lib.hbl_peak_mfma(kind, ctypes.c_void_p(sink.data_ptr()), sink.numel(), blocks, iters, sp), "mfma")
        ops = lib.hbl_peak_mfma_ops(kind, blocks, iters)
        out[key] = round(ops / (best_us(run, reps=2) * 1e-6) / 1e12, 1)
    del sink
    # the data path of one compute unit: one 8-wave workgroup per compute unit, a 2 MiB source that the L2
    # caches hold; cycles from the shader clock the probe reads (s_memtime against the 100 MHz counter)
    lib.hbl_peak_lds.argtypes = [I32, P, I64, I32, I32, P, I64, P, I64, P]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    lsrc = torch.ones((2 << 20) // 4, dtype=torch.int32, device=dev)
    clk = torch.zeros(2 * cus, dtype=torch.int64, device=dev)
    lsink = torch.zeros(cus, dtype=torch.int32, device=dev)
    rounds = 2000
    for kind, key in ((0, "lds_read"), (1, "lds_direct"), (2, "fp6_kstep"), (3, "fp6_kstep_nobarrier"),
                      (4, "fp6_kstep_noload")):
        def run(kind=kind):
            ok(lib.hbl_peak_lds(kind, ctypes.c_void_p(lsrc.data_ptr()), lsrc.numel() * 4, cus, rounds,
                                ctypes.c_void_p(clk.data_ptr()), clk.numel(), ctypes.c_void_p(lsink.data_ptr()),
                                lsink.numel(), sp), "lds")
        us = best_us(run, reps=1)
        c = clk.view(cus, 2).double().cpu()
        ghz = float(c[:, 0].median() / (c[:, 1].median() / 100e6) / 1e9)
        cyc = us * 1e3 * ghz / rounds  # shader cycles per round
        if kind == 0:
            out["lds_read_B_per_clk_cu"] = round(8 * 14 * 1024 / cyc, 1)
        elif kind == 1:
            out["lds_direct_load_B_per_clk_cu"] = round(8 * 5 * 1024 / cyc, 1)
        else:  # per SIMD and round: 2 waves x 16 instructions at 32 cycles each at the dense rate
            out[key + "_mfma_util"] = round(2 * 16 * 32 / cyc, 4)
            out[key + "_clock_GHz"] = round(ghz, 3)
    del lsrc, clk, lsink
    torch.cuda.synchronize()
    out["method"] = ("512 MiB 16-byte streaming copy (2 x bytes); 8 MiB and 64 MiB streaming reads and an empty "
                     "256-block kernel, graph-replayed; 2048 x 256-thread blocks each issuing 4 independent "
                     "matrix-core instructions per round on register operands; one 8-wave workgroup per compute "
                     "unit for the LDS data path: per wave and round 14 LDS reads of 16 B (lds_read), 5 LDS-direct "
                     "loads of 1 KiB from a 2 MiB source (lds_direct), and both with 16 FP6 x FP4 instructions "
                     "and a barrier (fp6_kstep: one K step of the 256 x 256 FP6 x FP4 tile; _nobarrier without the "
                     "barrier, _noload without the loads); a 32 MiB streaming write, graph-replayed")
    _PEAKS = out
    log("measured peaks done")
    return out


def with_measured_peak(roof, key):
    """Add the measured ceiling for this roofline's bound and the fraction of it."""
    pk = measured_peaks()
    roof["peak_measured"] = pk[key]
    roof["peak_measured_key"] = key
    roof["frac_measured"] = round(roof["achieved"] / pk[key], 4)
    return roof


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="chain_3b",
                   help="chain_3b (default: the 3B-like four-layer chain) or one layer of workloads/")
    p.add_argument("--layer", default=None, help="alias of --workload for one layer")
    p.add_argument("--op", choices=("layer", "heads", "backward", "base3"), default="layer",
                   help="layer: the H-BitLinear forward (default); heads: the low-bit attention-state quantiser "
                        "(per-head absmax to a 3-bit KV cache) on the 3B-like KV shape; backward: the layer's "
                        "straight-through backward (dX and dW) on --layer; base3: decode with base-3 weights")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-subresults", action="store_true", help="skip the other workloads' figures")
    p.add_argument("--kernel-iters", type=int, default=20)
    p.add_argument("--counter-run", action="store_true",
                   help="for rocprofv3 --pmc passes: a 256 MiB device copy (the counters' known-size reference), "
                        "then each kernel of the workload 3 times; prints no JSON")
    return p.parse_args()


def read_kv(path):
    """Parse a 'key = value' text file (lines starting with # are comments)."""
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#") and "=" in line:
                k, v = line.split("=", 1)
                out[k.strip()] = v.strip()
    return out


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel, workload):
    """HBM bytes per launch from committed counter passes (profiles/), only
    while the kernel's sources are unchanged since the counters were taken."""
    tfile = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (kernel, workload))
    if not os.path.exists(tfile):
        return None
    t = read_kv(tfile)
    if t.get("source_hash") != source_hash(t.get("sources", "").split()):
        return None
    return int(t["bytes_per_launch"])


# ------------------------------------------------------------------ setup --
def _to_dev(X):
    import numpy as np
    import torch
    if X.dtype == np.uint16:
        return torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(X).to("cuda:0")


def _use_fp4(layer):
    """INT4 prefill layers run on the FP6 x FP4 matrix cores with FP4 weights."""
    import bit_bitlinear_amd as hbl
    cfg = hbl.Config(act_bits=layer.act_bits, hadamard=layer.hadamard)
    return layer.act_bits == 4 and layer.M > 64 and layer.K >= 512 and \
        hbl.hbl_forward_workspace_bytes(layer.M, layer.K, layer.N, cfg) > hbl.hbl_workspace_bytes(layer.M, layer.K, cfg)


class Prepared:
    """One layer's device buffers: R rotating sets of (X, weights, workspace, Y)."""

    def __init__(self, layer, seed=0, rotate=True):
        import torch

        import bit_bitlinear_amd as hbl
        import workloads
        self.layer = L = layer
        self.cfg = hbl.Config(act_bits=L.act_bits, hadamard=L.hadamard)
        self.fp4 = _use_fp4(L)
        self.X_host, self.W_host, _ = workloads.make_inputs(L, seed)
        X = _to_dev(self.X_host)
        Wd = torch.from_numpy(self.W_host).to("cuda:0")
        self.ydt = torch.bfloat16 if L.y_dtype == "bf16" else torch.float32
        # weights: ternarised once (S0), then converted to FP4 for the FP6 x FP4 path
        self.wws = torch.empty(hbl.hbl_weight_workspace_bytes(L.N, L.K), dtype=torch.uint8, device="cuda:0")
        self.Wlat = Wd
        Wp, alpha = hbl.hbl_quantize_weights(Wd, 1e-5, ws=self.wws)
        W4 = hbl.hbl_pack_fp4(Wp, L.K) if self.fp4 else None
        self.alpha = alpha
        # the workspace of the fastest forward path
        ws_bytes = (hbl.hbl_forward_fp4_workspace_bytes(L.M, L.K, self.cfg) if self.fp4
                    else hbl.hbl_forward_workspace_bytes(L.M, L.K, L.N, self.cfg))
        y_bytes = L.M * L.N * (2 if self.ydt == torch.bfloat16 else 4)
        w_bytes = L.N * L.K // 2 if self.fp4 else L.N * L.K // 4
        set_bytes = X.numel() * X.element_size() + w_bytes + ws_bytes + y_bytes
        self.set_bytes = set_bytes
        self.R = max(1, -(-ROTATE_BYTES // set_bytes)) if rotate else 1
        self.sets = []
        for r in range(self.R):
            s = {"X": X if r == 0 else X.clone(),
                 "Wp": Wp if r == 0 else Wp.clone(),
                 "ws": torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda:0"),
                 "Y": torch.empty((L.M, L.N), dtype=self.ydt, device="cuda:0")}
            if self.fp4:
                s["W4"] = W4 if r == 0 else W4.clone()
            self.sets.append(s)
        del Wd
        torch.cuda.synchronize()

    def forward(self, r):
        import bit_bitlinear_amd as hbl
        s, L = self.sets[r], self.layer
        if self.fp4:
            hbl.hbl_forward_fp4(s["X"], s["W4"], self.alpha, L.N, self.cfg, Y=s["Y"], ws=s["ws"])
        else:
            hbl.hbl_forward(s["X"], s["Wp"], self.alpha, L.N, self.cfg, Y=s["Y"], ws=s["ws"])

    # the stage entry points, writing into the same workspace regions as the forward
    def stage_views(self, r):
        import torch
        L, s = self.layer, self.sets[r]
        if self.fp4:
            cb = -(-(L.M * L.K * 3 // 4) // 256) * 256
            codes = s["ws"][:L.M * L.K * 3 // 4].view(L.M, L.K * 3 // 4)
        else:
            cb = -(-(L.M * L.K * L.act_bits // 8) // 256) * 256
            codes = s["ws"][:L.M * L.K * L.act_bits // 8].view(L.M, -1)
            if L.act_bits == 8:
                codes = codes.view(torch.int8)
        xs = s["ws"][cb:cb + 4 * L.M].view(torch.float32)
        return codes, xs

    def act(self, r):
        import bit_bitlinear_amd as hbl
        codes, xs = self.stage_views(r)
        if self.fp4:
            hbl.hbl_quantize_activations_fp6(self.sets[r]["X"], self.cfg, codes6=codes, xscale=xs)
        else:
            hbl.hbl_quantize_activations(self.sets[r]["X"], self.cfg, codes=codes, xscale=xs)

    def gemm(self, r):
        import bit_bitlinear_amd as hbl
        L, s = self.layer, self.sets[r]
        codes, xs = self.stage_views(r)
        if self.fp4:
            hbl.hbl_gemm_fp6fp4(codes, xs, L.K, s["W4"], self.alpha, L.N, Y=s["Y"])
        else:
            hbl.hbl_gemm(codes, xs, L.act_bits, L.K, s["Wp"], self.alpha, L.N, Y=s["Y"])

    def work(self):
        """Algorithmic work per launch of each kernel: bytes that must cross HBM
        (input rows, INT8/INT4-equivalent codes, scales, 2-bit weights, output)
        and 2*M*N*K integer ops for the product."""
        L = self.layer
        x_bytes = L.M * L.K * (2 if L.x_dtype == "bf16" else 4)
        y_bytes = L.M * L.N * (2 if L.y_dtype == "bf16" else 4)
        code_bytes = L.M * L.K * L.act_bits // 8
        return {"act_bytes": x_bytes + code_bytes + 4 * L.M,
                "gemm_ops": 2 * L.M * L.N * L.K,
                "gemm_bytes": code_bytes + 4 * L.M + L.N * L.K // 4 + y_bytes,
                "fwd_small_bytes": x_bytes + L.N * L.K // 4 + 4 + y_bytes}


def capture(fns):
    """One HIP graph per entry of fns (each a callable queueing launches)."""
    import torch
    graphs = []
    for f in fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            f()
        graphs.append(g)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    return graphs


def replay_timed(graphs, n):
    """Replay graphs[i % R] for i < n; returns (wall seconds, event ms), both
    bracketed by synchronisations."""
    import torch
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(n):
        graphs[i % len(graphs)].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1)


def graph_us(fn, R, iters):
    """Microseconds per call of fn(r): one HIP graph holding fn(0) .. fn(R-1)
    (one call per buffer set, so short kernels run back to back without the
    host in between), replayed ceil(iters / R) times; events on the launch
    stream."""
    graphs = capture([lambda: [fn(r) for r in range(R)]])
    reps = max(1, -(-iters // R))
    # untimed replays first: the first replays of a freshly prepared layer
    # run up to a fifth slower (measured on the 7B Wdown forward: 417 us on
    # the first timing, 338 us on the next)
    replay_timed(graphs, max(2, reps // 2))
    _, ms = replay_timed(graphs, reps)
    del graphs
    return ms * 1e3 / (reps * R)


def roofline(kernel, bound, work, us, unit, peak, peak_key, traffic=None, desc=""):
    per_s = work / (us * 1e-6)
    achieved = per_s / 1e12 if unit == "TFLOP/s" else per_s / 1e9
    r = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic, "work_per_launch": work,
         "us_per_launch": round(us, 3), "work_desc": desc}
    return with_measured_peak(r, peak_key)


# ------------------------------------------------------------- the chain --
def bench_chain(args):
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    torch.cuda.set_device(0)
    hbl.load_library()
    layers = workloads.CHAIN_3B
    M = layers[0].M
    preps = []
    for i, L in enumerate(layers):
        preps.append(Prepared(L, seed=i, rotate=False))
        log("inputs ready: %s" % L.desc)
    assert all(p.fp4 for p in preps)
    step_bytes = sum(p.set_bytes for p in preps)
    R = max(1, -(-ROTATE_BYTES // step_bytes))
    if R > 1:  # a small chain would need more sets; the 3B chain's step touches > 1 GiB
        raise RuntimeError("chain smaller than the rotation size")

    stream = torch.cuda.current_stream()

    def step(evs=None):
        # one forward of each layer: its two launches (the activation kernel,
        # then the GEMM: exactly the launches of hbl_forward_fp4), with HIP
        # events on the launch stream around each when evs is given
        for j, p in enumerate(preps):
            if evs is not None:
                evs[j][0].record(stream)
            p.act(0)
            if evs is not None:
                evs[j][1].record(stream)
            p.gemm(0)
            if evs is not None:
                evs[j][2].record(stream)

    for _ in range(args.warmup):
        step()
    # the timed region: exactly --steps steps, launched back to back (the host
    # enqueues a step in well under the GPU's time for it), every kernel
    # bracketed by events, so the per-kernel averages come from these steps
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in preps] for _ in range(args.steps)]
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(ev[i])
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e_start.elapsed_time(e_end)
    ms_per_step = wall / args.steps * 1e3
    log("chain: %d steps timed, %.3f ms per step" % (args.steps, ms_per_step))
    ops_step = sum(2 * p.layer.M * p.layer.N * p.layer.K for p in preps)
    # cross-check: the same steps through hbl_forward_fp4, replayed from a HIP graph
    graphs = capture([lambda r=0: [p.forward(0) for p in preps]])
    wall_g, _ = replay_timed(graphs, args.steps)
    del graphs

    per_layer = []
    n_it = args.steps
    for j, p in enumerate(preps):
        t_act = sum(ev[i][j][0].elapsed_time(ev[i][j][1]) for i in range(n_it)) / n_it * 1e3
        t_gemm = sum(ev[i][j][1].elapsed_time(ev[i][j][2]) for i in range(n_it)) / n_it * 1e3
        w = p.work()
        L = p.layer
        act6_bytes = L.M * L.K * 2 + L.M * L.K * 3 // 4 + 4 * L.M
        per_layer.append({
            "layer": L.desc, "act_us": round(t_act, 3), "gemm_us": round(t_gemm, 3),
            "gemm_ops": w["gemm_ops"], "gemm_TOPS": round(w["gemm_ops"] / (t_gemm * 1e-6) / 1e12, 1),
            "gemm_frac_f6f4_peak": round(w["gemm_ops"] / (t_gemm * 1e-6) / 1e12 / PEAK_F6F4_TOPS, 4),
            "act_GBps": round(w["act_bytes"] / (t_act * 1e-6) / 1e9, 1),
            "act_bytes_algorithmic": w["act_bytes"], "act_bytes_fp6": act6_bytes})
    # weight preparation (S0 + FP4 conversion), once per weight, timed apart
    wprep = []
    for p in preps:
        L = p.layer
        t_wq = graph_us(lambda r, p=p: hbl.hbl_quantize_weights(p.Wlat, 1e-5, W_packed=p.sets[0]["Wp"],
                                                                 alpha=p.alpha, ws=p.wws), 1, 3)
        t_f4 = graph_us(lambda r, p=p: hbl.hbl_pack_fp4(p.sets[0]["Wp"], L.K, W4=p.sets[0]["W4"]), 1, 3)
        wprep.append({"layer": L.name, "ternarise_us": round(t_wq, 2), "to_fp4_us": round(t_f4, 2),
                      "ternarise_GBps": round((L.N * L.K * 4 + L.N * L.K // 4 + 4) / (t_wq * 1e-6) / 1e9, 1)})
    tot_gemm_us = sum(x["gemm_us"] for x in per_layer)
    tot_act_us = sum(x["act_us"] for x in per_layer)
    n_l = len(preps)
    # the dominant kernel: the FP6 x FP4 GEMM, one launch per layer; its
    # average launch does (ops of the four layers) / 4 in (their time) / 4
    traffic = committed_traffic("gemm_f6f4", "chain_3b")
    roof = roofline("gemm_f6f4_kernel (hbl_gemm_fp6fp4; one launch per layer, averaged over the 4 layers)",
                    "mfma", ops_step // n_l, tot_gemm_us / n_l, "TFLOP/s", PEAK_F6F4_TOPS, "mfma_f6f4_TFLOPS",
                    traffic, "2*M*N*K ops of the 4 layers / 4 per launch; INT4 codes as FP6 E3M2 x ternary "
                             "weights as FP4 E2M1, exact fp32 sums")
    del preps
    torch.cuda.empty_cache()

    log("chain: per-kernel times and weight preparation done")
    subs = None if args.no_subresults else subresults(args)
    cpu = None if args.no_cpu_baseline else cpu_baseline_chain(layers)
    if cpu:
        log("cpu baseline done")
    out = {
        "metric": METRIC,
        "value": round(M * args.steps / wall, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6xfp4",
        "data": "synthetic (seeded Gaussian, outlier-mixture and SwiGLU-like activations; N(0,0.02) latent "
                "weights, ternarised once)",
        "config": {"workload": "chain_3b: 3B-like layer chain at 8192 tokens, INT4 activations, bf16 in/out: "
                               "QKV 4096->12288 and gate/up 4096->32768 (BitLinear), Wo 4096->4096 and Wdown "
                               "16384->4096 (H-BitLinear)",
                   "M": M, "layers": [p["layer"] for p in per_layer], "act_bits": 4,
                   "step": "the forward of each of the 4 layers (hbl_quantize_activations_fp6: norm [+ Hadamard] "
                           "+ INT4 codes as FP6; hbl_gemm_fp6fp4: FP6 x FP4 GEMM + rescale; the two launches of "
                           "hbl_forward_fp4) against weights ternarised and converted to FP4 once",
                   "timing": "exactly --steps steps launched back to back, HIP events around every kernel on the "
                             "launch stream; the roofline's kernel times are averages over these steps"},
        "tops": round(ops_step * args.steps / wall / 1e12, 2),
        "ms_per_step_events": round(ev_ms / args.steps, 5),
        "ms_per_step_graph": round(wall_g / args.steps * 1e3, 5),
        "kernel_us_per_step": {"gemm_f6f4": round(tot_gemm_us, 2), "act_fp6": round(tot_act_us, 2)},
        "roofline": roof,
        "layers": per_layer,
        "weight_prep": wprep,
        "box_peaks": measured_peaks(),
        "subresults": subs,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def subresults(args):
    """The other workloads, each measured the same way (graph replay over
    rotating buffer sets): the forward, and its dominant kernel against its
    roofline."""
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    out = {}
    it = max(20, args.kernel_iters)
    for layer in (workloads.WO_1P3B, workloads.WDOWN_7B) + workloads.DECODE:
        p = Prepared(layer)
        L, w = p.layer, p.work()
        fwd = graph_us(p.forward, p.R, it)
        r = {"workload": L.desc, "forward_us": round(fwd, 3), "tokens_per_s": round(L.M / (fwd * 1e-6), 1),
             "forward_TOPS": round(w["gemm_ops"] / (fwd * 1e-6) / 1e12, 2),
             "gemm": "FP6 x FP4 matrix cores" if p.fp4 else "INT8 matrix cores" if L.M > 64 else "decode GEMV"}
        fused = L.M == 1 and 1024 <= L.K <= 16384
        if fused:
            # one launch (Kernel F): the forward is the kernel
            r["roofline"] = roofline("forward_small_kernel (hbl_forward, one launch)", "hbm", w["fwd_small_bytes"],
                                     fwd, "GB/s", PEAK_HBM_GBS, "hbm_read_8MiB_GBps", None,
                                     "read X + 2-bit W + alpha, write Y")
        else:
            act = graph_us(p.act, p.R, it)
            gemm = graph_us(p.gemm, p.R, it)
            r["act_us"] = round(act, 3)
            r["act_GBps"] = round(w["act_bytes"] / (act * 1e-6) / 1e9, 1)
            r["gemm_us"] = round(gemm, 3)
            if p.fp4:
                r["roofline"] = roofline("gemm_f6f4_kernel (hbl_gemm_fp6fp4)", "mfma", w["gemm_ops"], gemm,
                                         "TFLOP/s", PEAK_F6F4_TOPS, "mfma_f6f4_TFLOPS",
                                         committed_traffic("gemm_f6f4", L.name), "2*M*N*K ops")
            elif L.M > 64:
                r["roofline"] = roofline("gemm_dma_kernel (hbl_gemm, INT8)", "mfma", w["gemm_ops"], gemm, "TFLOP/s",
                                         PEAK_I8_TOPS, "mfma_i8_TOPS", committed_traffic("gemm_i8_mfma", L.name),
                                         "2*M*N*K integer ops")
            else:
                # decode: hbl_forward = activation kernel (codes in the decode
                # tile layout) + decode GEMM; the bytes the forward must move
                # against its time
                r["roofline"] = roofline("hbl_forward (activation kernel + decode GEMM)", "hbm",
                                         w["fwd_small_bytes"], fwd, "GB/s", PEAK_HBM_GBS, "hbm_read_8MiB_GBps", None,
                                         "read X + 2-bit W + alpha, write Y (the codes are intermediate)")
                r["gemm_single_pass_us"] = r.pop("gemm_us")
        out[L.name] = r
        log("subresult %s: forward %.3f us" % (L.name, fwd))
        del p
        torch.cuda.empty_cache()
    return out


def cpu_baseline_chain(layers):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload: the forward of the first S rows of each of the four
    layers (weights ternarised once beforehand, as on the GPU), scaled to
    tokens/s = S / (time of the four layers)."""
    import oracle

    cores = oracle.num_threads()
    Wq = []
    t0 = time.perf_counter()
    inputs = []
    import workloads
    for i, L in enumerate(layers):
        X, W, _ = workloads.make_inputs(L, seed=i, M=64)
        q, _, a = oracle.quantize_weights(W)
        Wq.append((q, a))
        inputs.append(X)
    t_wq = time.perf_counter() - t0

    def run(S):
        t = time.perf_counter()
        for L, X, (q, a) in zip(layers, inputs, Wq):
            oracle.forward(X[:S], q, a, bits=L.act_bits, hadamard=L.hadamard)
        return time.perf_counter() - t

    per_row = run(cores) / cores
    S = int(max(cores, min(64, round(2.0 / max(per_row, 1e-6)))))
    S -= S % cores if S > cores else 0
    t = run(S)
    return {"value": round(S / t, 3), "unit": "tokens/s", "cores": cores, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": "forward of the first %d of %d rows through the 4 chain layers (%.2f s wall on %d OpenMP "
                      "threads; weights ternarised beforehand, %.1f s, not counted), scaled to tokens/s"
                      % (S, layers[0].M, t, cores, t_wq),
            "cpu_seconds": round(t * cores, 1)}


# -------------------------------------------------------------- one layer --
def bench_single(args, layer):
    """One layer of workloads/ as the step (forward with weights prepared once),
    for the profiles of that layer; the JSON line has the same fields."""
    import torch

    import bit_bitlinear_amd as hbl

    torch.cuda.set_device(0)
    hbl.load_library()
    p = Prepared(layer)
    L, w = p.layer, p.work()
    for i in range(args.warmup):
        p.forward(i % p.R)
    torch.cuda.synchronize()
    graphs = capture([lambda r=r: p.forward(r) for r in range(p.R)])
    replay_timed(graphs, max(2, args.warmup))  # untimed replays first (see graph_us)
    wall, ev_ms = replay_timed(graphs, args.steps)
    del graphs
    it = max(20, args.kernel_iters)
    fused = L.M == 1 and 1024 <= L.K <= 16384
    fwd = graph_us(p.forward, p.R, it)
    if fused:
        roof = roofline("forward_small_kernel (hbl_forward, one launch)", "hbm", w["fwd_small_bytes"], fwd, "GB/s",
                        PEAK_HBM_GBS, "hbm_read_8MiB_GBps", None, "read X + 2-bit W + alpha, write Y")
        kern = {}
    else:
        act = graph_us(p.act, p.R, it)
        gemm = graph_us(p.gemm, p.R, it)
        kern = {"act_us": round(act, 3), "gemm_us": round(gemm, 3),
                "act_GBps": round(w["act_bytes"] / (act * 1e-6) / 1e9, 1)}
        if p.fp4:
            roof = roofline("gemm_f6f4_kernel (hbl_gemm_fp6fp4)", "mfma", w["gemm_ops"], gemm, "TFLOP/s",
                            PEAK_F6F4_TOPS, "mfma_f6f4_TFLOPS", committed_traffic("gemm_f6f4", L.name),
                            "2*M*N*K ops")
        elif L.M > 64:
            roof = roofline("gemm_dma_kernel (hbl_gemm, INT8)", "mfma", w["gemm_ops"], gemm, "TFLOP/s",
                            PEAK_I8_TOPS, "mfma_i8_TOPS", committed_traffic("gemm_i8_mfma", L.name),
                            "2*M*N*K integer ops")
        else:
            roof = roofline("hbl_forward (activation kernel + decode GEMM)", "hbm",
                            w["fwd_small_bytes"], fwd, "GB/s", PEAK_HBM_GBS, "hbm_read_8MiB_GBps", None,
                            "read X + 2-bit W + alpha, write Y (the codes are intermediate)")
            kern["gemm_single_pass_us"] = kern.pop("gemm_us")
    # the same layer from latent weights (ternarised in every step), for training-time callers
    lat = None
    if not p.fp4:
        lat = graph_us(lambda r: hbl.hbl_forward_latent(p.sets[r]["X"], p.Wlat, p.cfg, 1e-5,
                                                        W_packed=p.sets[r]["Wp"], alpha=p.alpha, Y=p.sets[r]["Y"],
                                                        ws=p.sets[r]["ws"], wws=p.wws), p.R, it)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_chain((L,))
    print(json.dumps({
        "metric": METRIC, "value": round(L.M * args.steps / wall, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp6xfp4" if p.fp4 else "i8",
        "data": "synthetic (seeded; outlier-channel activations, N(0,0.02) latent weights, ternarised once)",
        "config": {"workload": L.desc, "M": L.M, "K": L.K, "N": L.N, "act_bits": L.act_bits,
                   "hadamard": L.hadamard, "rotating_sets": p.R,
                   "step": "hbl_forward_fp4" if p.fp4 else "hbl_forward",
                   "timing": "HIP graph replay, exactly --steps replays"},
        "tops": round(w["gemm_ops"] * args.steps / wall / 1e12, 2),
        "ms_per_step_events": round(ev_ms / args.steps, 5),
        "forward_us": round(fwd, 3), "latent_step_us": None if lat is None else round(lat, 3),
        "kernels": kern, "roofline": roof, "box_peaks": measured_peaks(), "cpu_baseline": cpu,
    }), flush=True)


def counter_run(name):
    """For rocprofv3 --pmc passes: a 256 MiB device copy (the counters'
    known-size reference), then each kernel of the workload 3 times."""
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    torch.cuda.set_device(0)
    hbl.load_library()
    layers = workloads.CHAIN_3B if name == "chain_3b" else (workloads.by_name(name),)
    src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    del src, dst
    for i, L in enumerate(layers):
        p = Prepared(L, seed=i, rotate=False)
        for _ in range(3):
            p.act(0)
            p.gemm(0)
            p.forward(0)
        torch.cuda.synchronize()
        del p
        torch.cuda.empty_cache()
    print("counter run done: %s" % name, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (every workload is one MI355X's share of a layer, and this build "
              "uses a single GPU); --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.op == "heads":
        return bench_heads(args)
    if args.op == "backward":
        if args.layer is None:
            args.layer = "wo_1.3b"
        return bench_backward(args)
    if args.op == "base3":
        if args.layer is None:
            args.layer = "decode_m1"
        return bench_base3(args)
    name = args.layer or args.workload
    if args.counter_run:
        return counter_run(name)
    if name == "chain_3b":
        return bench_chain(args)
    import workloads
    return bench_single(args, workloads.by_name(name))


def bench_backward(args):
    """The straight-through backward of --layer: one step = hbl_backward with
    bf16 dY (dX through the Hadamard and the norm, and dW).  Its contractions
    run on the bf16 matrix cores: dZ = alpha dY Wq (one contraction for a bf16
    dY) and dW = (dY d)^T q (high part and remainder, one launch with a
    contraction twice as long): 6 M N K flops."""
    import numpy as np
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    layer = workloads.by_name(args.layer)
    M, K, N, bits = layer.M, layer.K, layer.N, layer.act_bits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hbl.load_library()
    X, W, _ = workloads.make_inputs(layer, 0)
    rng = np.random.default_rng(1)
    dY = workloads.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    to_t = lambda a: (torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16
                      else torch.from_numpy(a)).to(dev)
    Xd, dYd = to_t(X), to_t(dY)
    cfg = hbl.Config(act_bits=bits, hadamard=layer.hadamard)
    Wp, alpha = hbl.hbl_quantize_weights(torch.from_numpy(W).to(dev))
    ws_bytes = hbl.hbl_backward_workspace_bytes(M, K, N, cfg, True)
    set_bytes = Xd.numel() * Xd.element_size() + dYd.numel() * 2 + ws_bytes + 4 * M * K + 4 * N * K
    R = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = [(Xd if r == 0 else Xd.clone(), dYd if r == 0 else dYd.clone(),
             torch.empty((M, K), dtype=torch.float32, device=dev), torch.empty((N, K), dtype=torch.float32, device=dev),
             torch.empty(ws_bytes, dtype=torch.uint8, device=dev)) for r in range(R)]

    def step(s):
        hbl.hbl_backward(s[1], s[0], Wp, alpha, cfg, dX=s[2], dW=s[3], ws=s[4])

    for i in range(max(2, args.warmup // 4)):
        step(sets[i % R])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            step(sets[r])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-max(R, args.steps // 4) // R))
    timed = reps * R
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / timed * 1e3
    flops = 6.0 * M * N * K
    achieved = flops / (us * 1e-6) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        S = 16
        Wq = oracle.unpack_ternary(Wp.cpu().numpy(), K)
        a = float(alpha.cpu().numpy()[0])
        t0 = time.perf_counter()
        oracle.backward(dY[:S], X[:S], Wq, a, bits=bits, hadamard=layer.hadamard)
        t = time.perf_counter() - t0
        cpu = {"value": round(S / t, 2), "unit": "tokens/s", "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
               "sample": "dX and dW of the first %d of %d rows (%.2f s, single-threaded C; dW of a row subset is "
                         "the same work per row)" % (S, M, t)}
    print(json.dumps({
        "metric": "H-BitLinear straight-through backward tokens/s (dX and dW)",
        "value": round(M * timed / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": timed,
        "warmup": max(2, args.warmup // 4), "ms_per_step": round(wall / timed * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (the layer's seeded inputs; dY ~ N(0,1) in bf16)",
        "config": {"workload": "backward of %s" % layer.desc, "M": M, "K": K, "N": N,
                   "rotating_sets": R, "timing": "HIP graph replay of captured launches"},
        "roofline": with_measured_peak({"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "gemm_bf16_dma_kernel (dZ, then dW with high part and remainder in one launch)", "us_per_step": round(us, 3),
                     "work_desc": "6 M N K flops of the three bf16 products over the whole step's time (the "
                                  "operand preparation and the row kernel included), a lower bound for the "
                                  "products alone"}, "mfma_bf16_TFLOPS"),
        "box_peaks": measured_peaks(),
        "cpu_baseline": cpu,
    }))


def bench_heads(args):
    """The low-bit attention-state quantiser: one step = hbl_quantize_heads over
    the post-RoPE K (or V) states of 8192 tokens x 32 heads x 128 (bf16) to
    3-bit codes; HBM-bound (reads 2 bytes, writes 3/8 byte per element)."""
    import numpy as np
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    name, M, H, D, bits = workloads.KV_3B
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hbl.load_library()
    rng = np.random.default_rng(0)
    X = workloads.head_states(rng, M, H, D)
    Xb = workloads.f32_to_bf16_bits(X)
    Xd = torch.from_numpy(Xb.view(np.int16)).view(torch.bfloat16).to(dev)
    set_bytes = Xd.numel() * 2 + M * H * D * bits // 8 + 4 * M * H
    R = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = [(Xd if r == 0 else Xd.clone(), torch.empty((M, H, D * bits // 8), dtype=torch.uint8, device=dev),
             torch.empty((M, H), dtype=torch.float32, device=dev)) for r in range(R)]

    def step(s):
        hbl.hbl_quantize_heads(s[0], H, bits, 1e-5, codes=s[1], scales=s[2])

    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            step(sets[r])
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, -(-args.steps // R))
    timed = reps * R
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = ev0.elapsed_time(ev1) / timed * 1e3   # per launch, events on the launch stream
    work = M * H * D * 2 + M * H * D * bits // 8 + 4 * M * H
    achieved = work / (us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        oracle.quantize_heads(Xb, bits, eps=1e-5)
        t = time.perf_counter() - t0
        cpu = {"value": round(M / t, 2), "unit": "tokens/s", "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
               "sample": "the whole workload (%d x %d heads x %d), single-threaded C, %.3f s" % (M, H, D, t)}
    print(json.dumps({
        "metric": "low-bit attention-state quantisation tokens/s (per-head absmax to a 3-bit KV cache)",
        "value": round(M * timed / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": timed,
        "warmup": args.warmup, "ms_per_step": round(wall / timed * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) with a log-normal scale per token and head)",
        "config": {"workload": "%s: %d tokens x %d heads x %d, bf16 in, %d-bit codes" % (name, M, H, D, bits),
                   "rotating_sets": R, "timing": "HIP graph replay of captured launches"},
        "roofline": with_measured_peak({"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "head_quant_kernel", "us_per_launch": round(us, 3),
                     "work_desc": "read X (bf16) + write codes + write scales, %d bytes per launch" % work},
            "hbm_copy_GBps"),
        "box_peaks": measured_peaks(),
        "cpu_baseline": cpu,
    }))


def _graph_us(step, R, reps):
    """Capture step(0..R-1) in one HIP graph; microseconds per step over reps
    replays (events on the launch stream)."""
    import torch
    for r in range(R):
        step(r)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for r in range(R):
            step(r)
    for _ in range(max(2, reps // 2)):  # untimed replays first (see graph_us)
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(reps):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return ev0.elapsed_time(ev1) / (reps * R) * 1e3, wall / (reps * R), g


def bench_base3(args):
    """Decode with the weights stored five per byte: one step = hbl_forward_base3
    of the decode layer's tokens (activation quantisation, then the base-3 GEMV)
    against weights packed once beforehand, as a deployment holds them.  The
    2-bit forward of the same tokens is timed beside it."""
    import numpy as np
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    layer = workloads.by_name(args.layer) if args.layer.startswith("decode_m") else workloads.DECODE[0]
    if layer.M > 4:              # the base-3 GEMV takes 1 to 4 tokens
        layer = workloads.DECODE[0]
    M, K, N, bits = layer.M, layer.K, layer.N, layer.act_bits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hbl.load_library()
    X, W, _ = workloads.make_inputs(layer, 0)
    Xd = torch.from_numpy(X).to(dev)
    cfg = hbl.Config(act_bits=bits, hadamard=layer.hadamard)
    Wp, alpha = hbl.hbl_quantize_weights(torch.from_numpy(W).to(dev))
    W3 = hbl.hbl_pack_base3(Wp, K)
    torch.cuda.synchronize()
    w3_bytes = W3.numel()
    R = max(2, -(-ROTATE_BYTES // (w3_bytes + Wp.numel())))
    W3s = [W3] + [W3.clone() for _ in range(R - 1)]
    Wps = [Wp] + [Wp.clone() for _ in range(R - 1)]
    ws = torch.empty(hbl.hbl_workspace_bytes(M, K, cfg), dtype=torch.uint8, device=dev)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    codes = torch.empty((M, K if bits == 8 else K // 2), dtype=torch.int8 if bits == 8 else torch.uint8, device=dev)
    xs = torch.empty(M, dtype=torch.float32, device=dev)
    hbl.hbl_quantize_activations(Xd, cfg, codes=codes, xscale=xs)
    reps = max(1, -(-args.steps // R))
    fwd_us, wall, g1 = _graph_us(lambda r: hbl.hbl_forward_base3(Xd, W3s[r], alpha, N, cfg, Y=Y, ws=ws), R, reps)
    gemv_us, _, g2 = _graph_us(lambda r: hbl.hbl_gemm_base3(codes, xs, bits, K, W3s[r], alpha, N, Y=Y), R, reps)
    fwd2_us, _, g3 = _graph_us(lambda r: hbl.hbl_forward(Xd, Wps[r], alpha, N, cfg, Y=Y, ws=ws), R, reps)
    gemv2_us, _, g4 = _graph_us(lambda r: hbl.hbl_gemm(codes, xs, bits, K, Wps[r], alpha, N, Y=Y), R, reps)
    work = w3_bytes + M * K * bits // 8 + 4 * M + 4 + M * N * 2
    achieved = work / (gemv_us * 1e-6) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        Wq = oracle.unpack_base3(W3.cpu().numpy(), K)
        oracle.forward(X, Wq, float(alpha.cpu().numpy()[0]), bits=bits, hadamard=layer.hadamard)
        t = time.perf_counter() - t0
        cpu = {"value": round(M / t, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "cpu_model": cpu_model(),
               "kind": "oracle",
               "sample": "all %d tokens: base-3 unpack of the weights and the forward (%.2f s)" % (M, t)}
    print(json.dumps({
        "metric": "decode tokens/s with base-3 weights (five per byte)",
        "value": round(M / wall, 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps * R, "warmup": R,
        "ms_per_step": round(wall * 1e3, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8", "data": "synthetic (the decode layer's seeded inputs)",
        "config": {"workload": "%s with base-3 weights (%d bytes against %d in the 2-bit format)"
                               % (layer.desc, w3_bytes, Wp.numel()), "M": M, "K": K, "N": N,
                   "rotating_sets": R, "timing": "HIP graph replay of captured launches"},
        "forward_us": round(fwd_us, 3), "forward_2bit_us": round(fwd2_us, 3),
        "gemv_us": round(gemv_us, 3), "gemv_2bit_us": round(gemv2_us, 3),
        "roofline": with_measured_peak({"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "kernel": "gemv_base3_kernel", "us_per_launch": round(gemv_us, 3),
                     "work_desc": "base-3 weights + codes + scales + bf16 Y, %d bytes per launch" % work},
            "hbm_copy_GBps"),
        "box_peaks": measured_peaks(),
        "cpu_baseline": cpu,
    }))
    del g1, g2, g3, g4



if __name__ == "__main__":
    main()
