"""Seeded random forward configurations through the C ABI, against the
oracle: token counts from 1 to a few thousand (every dispatch path: the
one-token fused kernel, the small-M GEMV, the decode tiles, 64-row and full
GEMM tiles), every row length, INT4/INT8, with and without the Hadamard,
each norm, gain or none, both input and output dtypes.  Up to 16 rows per
case are checked against the oracle (the dense Hadamard costs K^2 per row)."""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import (check_codes_end_to_end, check_codes_given_inputs, check_dw, check_y, check_z, fp4_library_order,
                    to_dev, to_host, unpack_codes, y_to_f32)

pytestmark = pytest.mark.gpu


def _configs(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    Ms = [1, 2, 3, 4, 5, 9, 16, 17, 40, 63, 64, 65, 100, 129, 257, 700, 1500, 3000]
    Ks = [256, 512, 1024, 2048, 4096, 8192, 16384]
    out = []
    for i in range(n):
        K = int(rng.choice(Ks, p=[0.16, 0.16, 0.18, 0.18, 0.14, 0.1, 0.08]))
        M = int(rng.choice(Ms))
        if K == 16384:
            M = min(M, 700)
        N = int(rng.integers(1, 97)) * 16
        out.append(dict(M=M, K=K, N=N, bits=int(rng.choice([4, 8])), had=bool(rng.random() < 0.7),
                        norm=int(rng.choice([hbl.HBL_NORM_RMS, hbl.HBL_NORM_LN, hbl.HBL_NORM_NONE])),
                        gain=bool(rng.random() < 0.5), xdt=str(rng.choice(["f32", "bf16"])),
                        ydt=str(rng.choice(["f32", "bf16"])), big_ws=bool(rng.random() < 0.5), seed=i))
    return out


CONFIGS = _configs()


@pytest.mark.parametrize("c", CONFIGS, ids=lambda c: "M%d-K%d-N%d-a%d-h%d-n%d-g%d-%s-%s" % (
    c["M"], c["K"], c["N"], c["bits"], c["had"], c["norm"], c["gain"], c["xdt"], c["ydt"]))
def test_forward_random_config(c):
    import torch
    M, K, N, bits, had, norm = c["M"], c["K"], c["N"], c["bits"], c["had"], c["norm"]
    print("[case] random forward %s" % sorted(c.items()), flush=True)
    rng = np.random.default_rng(1000 + c["seed"])
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(1.5)).astype(np.float32)
    Xh = workloads.f32_to_bf16_bits(X) if c["xdt"] == "bf16" else X
    W = workloads.w_latent(rng, N, K)
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if c["gain"] else None
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm)
    ydt = torch.float32 if c["ydt"] == "f32" else torch.bfloat16
    Xd = to_dev(Xh)
    gd = None if gain is None else to_dev(gain)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    ws_bytes = hbl.hbl_forward_workspace_bytes(M, K, N, cfg) if c["big_ws"] else hbl.hbl_workspace_bytes(M, K, cfg)
    ws = torch.empty(max(1, ws_bytes), dtype=torch.uint8, device="cuda:0")
    Y = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=ydt, gain=gd, ws=ws)
    codes, xs, z, s = hbl.hbl_quantize_activations(Xd, cfg, gain=gd, z_debug=True, s_debug=True)
    torch.cuda.synchronize()
    rows = workloads.sample_rows(M, 16)
    a_gpu = to_host(alpha)[0]
    assert abs(float(a_gpu) - float(oracle.weight_alpha(W))) <= 1e-6 * float(oracle.weight_alpha(W))
    Wq = oracle.ternarize(W, a_gpu, 1e-5)
    assert np.array_equal(to_host(Wp), oracle.pack_ternary(Wq))
    q_gpu = unpack_codes(to_host(codes)[rows], K, bits)
    z_gpu, s_gpu, d_gpu = to_host(z)[rows], to_host(s)[rows], to_host(xs)[rows]
    ref = oracle.quantize_activations(Xh[rows], bits=bits, hadamard=had, gain=gain, norm=norm)
    check_z(z_gpu, ref["z"], "z")
    check_codes_given_inputs(z_gpu, s_gpu, d_gpu, q_gpu, bits, 0, 1e-5, "codes")
    check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], "end-to-end codes")
    # the forward's output is the oracle's product and rescale of the GPU's codes, bit for bit
    y_exact = oracle.rescale(oracle.int_gemm(q_gpu, Wq), d_gpu, a_gpu)
    got = to_host(Y)[rows]
    assert np.array_equal(got, y_exact if c["ydt"] == "f32" else oracle.f32_to_bf16(y_exact))
    # and, end to end, the oracle's own pipeline (boundary flips use the GPU's code)
    flipped = np.any(q_gpu != ref["q"], axis=1)
    q_cmp = np.where(flipped[:, None], q_gpu, ref["q"])
    check_y(y_to_f32(got), oracle.rescale(oracle.int_gemm(q_cmp, Wq), ref["d"], a_gpu), "y",
            bf16_out=c["ydt"] == "bf16")


def _bwd_configs(n=8, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        K = int(rng.choice([512, 1024, 2048, 4096, 8192]))
        out.append(dict(M=int(rng.choice([1, 7, 64, 65, 300, 1100])), K=K, N=int(rng.integers(1, 65)) * 16,
                        bits=int(rng.choice([4, 8])), had=bool(rng.random() < 0.7),
                        norm=int(rng.choice([hbl.HBL_NORM_RMS, hbl.HBL_NORM_LN, hbl.HBL_NORM_NONE])),
                        gain=bool(rng.random() < 0.5), dydt=str(rng.choice(["f32", "bf16"])),
                        xdt=str(rng.choice(["f32", "bf16"])), seed=i))
    return out


@pytest.mark.parametrize("c", _bwd_configs(), ids=lambda c: "M%d-K%d-N%d-a%d-h%d-n%d-g%d-%s-%s" % (
    c["M"], c["K"], c["N"], c["bits"], c["had"], c["norm"], c["gain"], c["dydt"], c["xdt"]))
def test_backward_random_config(c):
    """dX on up to 16 sampled rows (2e-5 of the row's largest value) and dW
    on 24 sampled columns (the bound of parity.check_dw) against the oracle."""
    import torch
    M, K, N, bits, had, norm = c["M"], c["K"], c["N"], c["bits"], c["had"], c["norm"]
    print("[case] random backward %s" % sorted(c.items()), flush=True)
    rng = np.random.default_rng(5000 + c["seed"])
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(1.5)).astype(np.float32)
    Xh = workloads.f32_to_bf16_bits(X) if c["xdt"] == "bf16" else X
    dY = rng.standard_normal((M, N)).astype(np.float32)
    dYh = workloads.f32_to_bf16_bits(dY) if c["dydt"] == "bf16" else dY
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if c["gain"] else None
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm)
    gd = None if gain is None else to_dev(gain)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(workloads.w_latent(rng, N, K)))
    dX, dW = hbl.hbl_backward(to_dev(dYh), to_dev(Xh), Wp, alpha, cfg, gain=gd)
    codes, _, _, _ = hbl.hbl_quantize_activations(to_dev(Xh), cfg, gain=gd)
    torch.cuda.synchronize()
    a = to_host(alpha)[0]
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    rows = workloads.sample_rows(M, 16)
    dX_ref, _ = oracle.backward(dYh[rows], Xh[rows], Wq, a, bits=bits, hadamard=had, gain=gain, norm=norm,
                                want_dW=False)
    got = to_host(dX)[rows].astype(np.float64)
    scale = np.maximum(np.max(np.abs(dX_ref), axis=1, keepdims=True), 1e-30)
    assert np.all(np.abs(got - dX_ref) <= 2e-5 * scale)
    cols = np.unique(np.concatenate([[0, K - 1], rng.choice(K, 22, replace=False)]))
    ref = oracle.quantize_activations(Xh, bits=bits, hadamard=had, gain=gain, norm=norm)
    q_gpu = unpack_codes(to_host(codes), K, bits)
    check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], "backward codes")
    qc = np.ascontiguousarray(np.where(q_gpu != ref["q"], q_gpu, ref["q"])[:, cols])
    dW_ref = oracle.weight_grad(dYh, qc, ref["d"])
    check_dw(to_host(dW)[:, cols], dYh, qc, ref["d"], dW_ref, "dW")


def _fp4_configs(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    Ms = [65, 100, 257, 700, 1500, 3000]
    Ks = [512, 1024, 2048, 4096, 8192, 16384]
    out = []
    for i in range(n):
        K = int(rng.choice(Ks))
        M = int(rng.choice(Ms)) if K < 16384 else int(rng.choice(Ms[:4]))
        N = int(rng.integers(1, 97)) * 16
        out.append(dict(M=M, K=K, N=N, had=bool(rng.random() < 0.7),
                        norm=int(rng.choice([hbl.HBL_NORM_RMS, hbl.HBL_NORM_LN, hbl.HBL_NORM_NONE])),
                        gain=bool(rng.random() < 0.5), xdt=str(rng.choice(["f32", "bf16"])),
                        ydt=str(rng.choice(["f32", "bf16"])), seed=i))
    return out


@pytest.mark.parametrize("c", _fp4_configs(), ids=lambda c: "M%d-K%d-N%d-h%d-n%d-g%d-%s-%s" % (
    c["M"], c["K"], c["N"], c["had"], c["norm"], c["gain"], c["xdt"], c["ydt"]))
def test_forward_fp4_random_config(c):
    """hbl_forward_fp4 (FP4 weights, FP6 codes) on random INT4 configurations:
    the FP4 bytes against the oracle, Y bit for bit equal to hbl_forward (INT8
    matrix-core path) and, on sampled rows, to the oracle's product and
    rescale of the GPU's codes."""
    import torch
    M, K, N, had, norm = c["M"], c["K"], c["N"], c["had"], c["norm"]
    print("[case] random forward_fp4 %s" % sorted(c.items()), flush=True)
    rng = np.random.default_rng(2000 + c["seed"])
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(1.5)).astype(np.float32)
    Xh = workloads.f32_to_bf16_bits(X) if c["xdt"] == "bf16" else X
    W = workloads.w_latent(rng, N, K)
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if c["gain"] else None
    cfg = hbl.Config(act_bits=4, hadamard=had, norm=norm)
    ydt = torch.float32 if c["ydt"] == "f32" else torch.bfloat16
    Xd = to_dev(Xh)
    gd = None if gain is None else to_dev(gain)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    W4 = hbl.hbl_pack_fp4(Wp, K)
    Y4 = hbl.hbl_forward_fp4(Xd, W4, alpha, N, cfg, y_dtype=ydt, gain=gd)
    ws = torch.empty(max(1, hbl.hbl_workspace_bytes(M, K, cfg)), dtype=torch.uint8, device="cuda:0")
    Y8 = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=ydt, gain=gd, ws=ws)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg, gain=gd)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(W4).reshape(-1), fp4_library_order(oracle.pack_fp4(oracle.unpack_ternary(to_host(Wp), K))))
    assert np.array_equal(to_host(Y4), to_host(Y8)), "FP6 x FP4 forward differs from the INT8 path"
    rows = workloads.sample_rows(M, 16)
    a_gpu = to_host(alpha)[0]
    Wq = oracle.ternarize(W, a_gpu, 1e-5)
    q_gpu = unpack_codes(to_host(codes)[rows], K, 4)
    y_exact = oracle.rescale(oracle.int_gemm(q_gpu, Wq), to_host(xs)[rows], a_gpu)
    got = to_host(Y4)[rows]
    assert np.array_equal(got, y_exact if c["ydt"] == "f32" else oracle.f32_to_bf16(y_exact))
