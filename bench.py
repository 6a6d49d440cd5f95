"""Benchmark of the H-BitLinear forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layer NAME] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch of synthetic input:
per-tensor absmean ternarisation of the latent weights and the layer forward
(norm + Hadamard + per-token quantisation, then the integer GEMM with the
rescale epilogue), run as hbl_forward_latent, which gives the results of
hbl_quantize_weights followed by hbl_forward bit for bit in three launches
(the same two calls are timed too, as ms_per_step_two_calls).  The default layer is the
attention output projection Wo of a 1.3B-like model: 4096 tokens, K = N = 2048,
bf16 activations, INT8 codes, bf16 output.  Inputs are seeded synthetic arrays
already resident in HBM; the timed steps rotate over enough distinct buffer
sets (> 512 MiB) that the 256 MB last-level cache cannot hold them.

Prints one JSON line.  Besides the throughput it reports, for the kernel that
takes the most time per step, the algorithmic work per launch divided by its
average launch time (HIP events on the launch stream) against the MI355X
peak and against the ceiling measured in the same process by the probe
kernels of libhbl_peaks.so (an HBM copy and dense matrix-core loops), and the
CPU oracle timed on a bounded row sample on the host cores.
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PEAK_I8_TOPS = 5000.0          # MI355X dense INT8 MFMA, TOP/s
PEAK_F6F4_TOPS = 10100.0       # MI355X dense FP6 / FP4 MFMA, TFLOP/s
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
ROTATE_BYTES = 576 << 20       # > 2 x 256 MB last-level cache

_PEAKS = None


def measured_peaks():
    """Ceilings measured on this GPU by the probe kernels of libhbl_peaks.so
    (built beside libhbl.so): a 512 MiB streaming copy (read + write bytes)
    and loops of dense i8, FP6 x FP4 and bf16 matrix-core instructions on
    register operands; each the best of 3 timed rounds after a warm-up, with
    HIP events on the stream the probes run on.  Computed once per process."""
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
    lib.hbl_peak_mfma.argtypes = [I32, P, I64, I32, I32, P]
    lib.hbl_peak_mfma_ops.argtypes = [I32, I32, I32]
    lib.hbl_peak_mfma_ops.restype = I64
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

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

    nbytes = 512 << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)

    def copy():
        if lib.hbl_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes, sp) != 0:
            raise RuntimeError("hbl_peak_copy failed")

    out = {"hbm_copy_GBps": round(2 * nbytes / (best_us(copy) * 1e-6) / 1e9, 1)}
    del src, dst
    blocks, iters = 2048, 2000
    sink = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    for kind, key in ((0, "mfma_i8_TOPS"), (1, "mfma_f6f4_TFLOPS"), (2, "mfma_bf16_TFLOPS")):
        def run(kind=kind):
            if lib.hbl_peak_mfma(kind, ctypes.c_void_p(sink.data_ptr()), sink.numel(), blocks, iters, sp) != 0:
                raise RuntimeError("hbl_peak_mfma failed")
        ops = lib.hbl_peak_mfma_ops(kind, blocks, iters)
        out[key] = round(ops / (best_us(run, reps=2) * 1e-6) / 1e12, 1)
    torch.cuda.synchronize()
    out["method"] = ("512 MiB 16-byte streaming copy (2 x bytes); 2048 x 256-thread blocks each issuing 4 "
                     "independent matrix-core instructions per round on register operands")
    _PEAKS = out
    return out


def with_measured_peak(roof, key):
    """Add the measured ceiling for this roofline's bound and the fraction of it."""
    pk = measured_peaks()
    roof["peak_measured"] = pk[key]
    roof["frac_measured"] = round(roof["achieved"] / pk[key], 4)
    return roof


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=400)
    p.add_argument("--warmup", type=int, default=40)
    p.add_argument("--layer", default="wo_1.3b")
    p.add_argument("--op", choices=("layer", "heads", "backward", "base3"), default="layer",
                   help="layer: the H-BitLinear step (default); heads: the low-bit attention-state quantiser "
                        "(per-head absmax to a 3-bit KV cache) on the 3B-like KV shape; backward: the layer's "
                        "straight-through backward (dX and dW) on --layer")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--kernel-iters", type=int, default=200)
    p.add_argument("--counter-run", action="store_true",
                   help="for rocprofv3 --pmc passes: a 256 MiB device copy (the counters' known-size reference), "
                        "then each kernel of the layer 3 times; prints no JSON")
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


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only (each workload is one MI355X's share of a layer); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_bitlinear_amd as hbl
    import workloads

    if args.op == "heads":
        return bench_heads(args)
    if args.op == "backward":
        return bench_backward(args)
    if args.op == "base3":
        return bench_base3(args)
    layer = workloads.by_name(args.layer)
    M, K, N, bits = layer.M, layer.K, layer.N, layer.act_bits
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hbl.load_library()

    # ---------------------------------------------------------------- inputs
    X, W, _ = workloads.make_inputs(layer, seed=0)
    if layer.x_dtype == "bf16":
        Xd = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        Xd = torch.from_numpy(X).to(dev)
    Wd = torch.from_numpy(W).to(dev)
    ydt = torch.bfloat16 if layer.y_dtype == "bf16" else torch.float32
    cfg = hbl.Config(act_bits=bits, hadamard=layer.hadamard)
    # the workspace that selects the fastest forward path (FP6 x FP4 matrix
    # cores for INT4 prefill shapes, else the INT8 ones)
    ws_bytes = hbl.hbl_forward_workspace_bytes(M, K, N, cfg)
    f6f4 = ws_bytes > hbl.hbl_workspace_bytes(M, K, cfg)
    wws_bytes = hbl.hbl_weight_workspace_bytes(N, K)
    y_bytes = M * N * (2 if ydt == torch.bfloat16 else 4)
    set_bytes = Xd.numel() * Xd.element_size() + Wd.numel() * 4 + N * K // 4 + ws_bytes + y_bytes
    R = max(2, -(-ROTATE_BYTES // set_bytes))
    sets = []
    for r in range(R):
        s = {
            "X": Xd if r == 0 else Xd.clone(),
            "W": Wd if r == 0 else Wd.clone(),
            "Wp": torch.empty((N, K // 4), dtype=torch.uint8, device=dev),
            "alpha": torch.empty(1, dtype=torch.float32, device=dev),
            "wws": torch.empty(wws_bytes, dtype=torch.uint8, device=dev),
            "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
            "Y": torch.empty((M, N), dtype=ydt, device=dev),
            "codes": torch.empty((M, K if bits == 8 else K // 2), dtype=torch.int8 if bits == 8 else torch.uint8,
                                 device=dev),
            "xs": torch.empty(M, dtype=torch.float32, device=dev),
        }
        sets.append(s)
    torch.cuda.synchronize()

    def step(s):
        hbl.hbl_forward_latent(s["X"], s["W"], cfg, 1e-5, W_packed=s["Wp"], alpha=s["alpha"], Y=s["Y"], ws=s["ws"],
                               wws=s["wws"])

    def step_two_calls(s):
        hbl.hbl_quantize_weights(s["W"], 1e-5, W_packed=s["Wp"], alpha=s["alpha"], ws=s["wws"])
        hbl.hbl_forward(s["X"], s["Wp"], s["alpha"], N, cfg, Y=s["Y"], ws=s["ws"])

    if args.counter_run:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)   # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        s0 = sets[0]
        for _ in range(3):
            hbl.hbl_quantize_weights(s0["W"], 1e-5, W_packed=s0["Wp"], alpha=s0["alpha"], ws=s0["wws"])
            hbl.hbl_quantize_activations(s0["X"], cfg, codes=s0["codes"], xscale=s0["xs"])
            hbl.hbl_gemm(s0["codes"], s0["xs"], bits, K, s0["Wp"], s0["alpha"], N, Y=s0["Y"])
            hbl.hbl_forward(s0["X"], s0["Wp"], s0["alpha"], N, cfg, Y=s0["Y"], ws=s0["ws"])
        torch.cuda.synchronize()
        print("counter run done: %s" % layer.desc)
        return

    # ---------------------------------------------------------------- steps
    # Eager warmup (also initialises every kernel), then the timed work is
    # captured once in HIP graphs (one launch per rotating buffer set) and the
    # graphs are replayed, so the host's per-call overhead does not gate the
    # GPU; the graph holds kernel launches only.
    for i in range(args.warmup):
        step(sets[i % R])
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in range(R):
                fn(sets[r])
        g.replay()
        torch.cuda.synchronize()
        return g

    reps = max(1, -(-args.steps // R))
    timed_steps = reps * R

    def timed_replays(g):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    wall = timed_replays(capture(step))
    ms_per_step = wall / timed_steps * 1e3
    tokens_per_s = M * timed_steps / wall
    wall_two = timed_replays(capture(step_two_calls))

    # ------------------------------------------------------ per-kernel timing
    stream = torch.cuda.current_stream()

    def time_launches(fn, iters):
        g = capture(fn)
        reps_k = max(1, -(-iters // R))
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps_k):
            g.replay()
        ev1.record(stream)
        ev1.synchronize()
        return ev0.elapsed_time(ev1) / (reps_k * R) * 1e3   # microseconds per launch

    it = args.kernel_iters
    t_wq = time_launches(lambda s: hbl.hbl_quantize_weights(s["W"], 1e-5, W_packed=s["Wp"], alpha=s["alpha"],
                                                            ws=s["wws"]), it)
    t_act = time_launches(lambda s: hbl.hbl_quantize_activations(s["X"], cfg, codes=s["codes"], xscale=s["xs"]), it)
    t_gemm = time_launches(lambda s: hbl.hbl_gemm(s["codes"], s["xs"], bits, K, s["Wp"], s["alpha"], N, Y=s["Y"]), it)
    # one token with K a power of two in [1024, 16384]: hbl_forward is one fused launch
    fused = M == 1 and 1024 <= K <= 16384 and (K & (K - 1)) == 0
    # hbl_forward as a whole (up to 64 tokens its codes take the decode GEMM's tiled order)
    t_fwd = time_launches(lambda s: hbl.hbl_forward(s["X"], s["Wp"], s["alpha"], N, cfg, Y=s["Y"], ws=s["ws"]), it)

    x_bytes = M * K * (2 if layer.x_dtype == "bf16" else 4)
    code_bytes = M * K * bits // 8
    kernels = {
        "weight_ternarise": {"us": t_wq, "bound": "hbm", "unit": "GB/s",
                             "work": N * K * 4 + N * K // 4 + 4,
                             "work_desc": "read latent W once (fp32) + write 2-bit W + alpha"},
        "norm_fwht_quant": {"us": t_act, "bound": "hbm", "unit": "GB/s",
                            "work": x_bytes + code_bytes + 4 * M,
                            "work_desc": "read X + write codes + write xscale"},
        "gemm_i8_mfma" if M > 64 else "gemv_decode": {
            "us": t_gemm, "bound": "mfma" if M > 64 else "hbm", "unit": "TFLOP/s" if M > 64 else "GB/s",
            "work": 2 * M * N * K if M > 64 else code_bytes + 4 * M + N * K // 4 + M * N * 2,
            "work_desc": "2*M*N*K integer ops" if M > 64 else "read codes + xscale + 2-bit W, write Y"},
    }
    if f6f4:
        # the FP6 x FP4 GEMM runs only inside hbl_forward (with the FP6
        # activation kernel and the FP4 weight conversion): its ops over the
        # whole forward's time, a lower bound for the GEMM alone
        kernels["forward_fp6xfp4"] = {
            "us": t_fwd, "bound": "mfma", "unit": "TFLOP/s", "work": 2 * M * N * K, "peak": PEAK_F6F4_TOPS,
            "work_desc": "2*M*N*K ops over hbl_forward (FP6 activation codes, FP4 weights, FP6 x FP4 GEMM)"}
    if fused:
        kernels["forward_small_fused"] = {
            "us": t_fwd, "bound": "hbm", "unit": "GB/s",
            "work": x_bytes + N * K // 4 + 4 + M * N * (2 if ydt == torch.bfloat16 else 4),
            "work_desc": "read X + 2-bit W + alpha, write Y (codes stay on chip)"}
    for k, v in kernels.items():
        per_s = v["work"] / (v["us"] * 1e-6)
        v["achieved"] = per_s / 1e12 if v["unit"] == "TFLOP/s" else per_s / 1e9
        v["peak"] = v.get("peak") or (PEAK_I8_TOPS if v["unit"] == "TFLOP/s" else PEAK_HBM_GBS)
        v["frac"] = v["achieved"] / v["peak"]
    # the dominant kernel of the step (for a fused forward or the FP6 x FP4
    # path, the stage kernels it replaces are not in the step)
    replaced = ("norm_fwht_quant", "gemv_decode") if fused else ("norm_fwht_quant", "gemm_i8_mfma") if f6f4 else ()
    dom_name = max((k for k in kernels if k not in replaced), key=lambda k: kernels[k]["us"])
    dom = kernels[dom_name]

    # HBM bytes per launch from committed counter passes, only while the
    # kernel's sources are unchanged since the counters were taken
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic_%s_%s.txt" % (dom_name, layer.name))
    if os.path.exists(tfile):
        t = read_kv(tfile)
        if t.get("source_hash") == source_hash(t.get("sources", "").split()):
            traffic = int(t["bytes_per_launch"])

    roofline = {"kernel": dom_name, "bound": dom["bound"], "achieved": round(dom["achieved"], 2),
                "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["frac"], 4), "traffic": traffic,
                "work_per_launch": dom["work"], "work_desc": dom["work_desc"], "us_per_launch": round(dom["us"], 3)}
    with_measured_peak(roofline, "hbm_copy_GBps" if dom["unit"] == "GB/s" else
                       "mfma_f6f4_TFLOPS" if dom["peak"] == PEAK_F6F4_TOPS else "mfma_i8_TOPS")

    # ----------------------------------------------------------- CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layer, X, W)

    out = {
        "metric": "H-BitLinear tokens/s + TOPS (a4/a8 x ternary W) and % of HBM/MFMA roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6xfp4" if f6f4 else "i8",
        "data": "synthetic (seeded; outlier-channel activations, N(0,0.02) latent weights)",
        "config": {"workload": layer.desc, "M": M, "K": K, "N": N, "act_bits": bits,
                   "hadamard": layer.hadamard, "x_dtype": layer.x_dtype, "y_dtype": layer.y_dtype,
                   "step": "hbl_forward_latent (ternarise latent W + forward; = hbl_quantize_weights then "
                           "hbl_forward, bit for bit)", "rotating_sets": R,
                   "gemm": ("FP6 x FP4 matrix cores (INT4 codes as FP6 E3M2, ternary as FP4 E2M1, exact fp32 sums)"
                            if f6f4 else "INT8 matrix cores (int32 sums)"),
                   "timing": "HIP graph replay of captured launches"},
        "tops": round(2.0 * M * N * K * timed_steps / wall / 1e12, 2),
        "ms_per_step_two_calls": round(wall_two / timed_steps * 1e3, 5),
        "forward_us": round(t_fwd, 3),
        "forward_only_tokens_per_s": round(M / (t_fwd * 1e-6), 1),
        "roofline": roofline,
        "box_peaks": measured_peaks(),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                    for k, v in kernels.items()},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(layer, X, W):
    """The oracle as it stands, timed on the host cores on a bounded sample of
    the same workload: weight quantisation of the full W once, then the
    forward of the first S rows; tokens/s scales the row time to all M rows."""
    import numpy as np

    import oracle

    Xs = X
    t0 = time.perf_counter()
    Wq, _, alpha = oracle.quantize_weights(W)
    t_wq = time.perf_counter() - t0
    # calibrate on 16 rows, then size the sample for about 2 s of wall time
    t0 = time.perf_counter()
    oracle.forward(Xs[:16], Wq, alpha, bits=layer.act_bits, hadamard=layer.hadamard)
    per_row = (time.perf_counter() - t0) / 16
    S = int(min(layer.M, max(64, round(2.0 / max(per_row, 1e-6)))))
    S = max(16, S - S % 16)
    t0 = time.perf_counter()
    oracle.forward(Xs[:S], Wq, alpha, bits=layer.act_bits, hadamard=layer.hadamard)
    t_rows = time.perf_counter() - t0
    t_step = t_wq + t_rows * layer.M / S
    cores = oracle.num_threads()
    return {"value": round(layer.M / t_step, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": "full weight ternarisation once (%.3f s) + forward of the first %d of %d rows (%.3f s), "
                      "scaled to all rows; %d OpenMP threads" % (t_wq, S, layer.M, t_rows, cores),
            "cpu_seconds": round((t_wq + t_rows) * cores, 1)}


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
        cpu = {"value": round(S / t, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
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
        cpu = {"value": round(M / t, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
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
        cpu = {"value": round(M / t, 3), "unit": "tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
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
