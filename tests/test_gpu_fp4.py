"""The INT4 prefill path with FP4 weights (hbl_pack_fp4, hbl_forward_fp4 and
its two stages) through the C ABI.

The FP4 weight bytes must equal the oracle's O14 packing of the same ternary
values; hbl_forward_fp4 must equal hbl_forward (INT8 matrix cores, the
smaller workspace) bit for bit, and the oracle's arithmetic on sampled
columns; the two stages (FP6 codes, FP6 x FP4 GEMM) must reproduce
hbl_forward_fp4.  Small, ragged and full-size shapes.
"""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import fp4_library_order, to_dev, to_host, unpack_codes

pytestmark = pytest.mark.gpu


def _announce(msg):
    print("[case] " + msg, flush=True)


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("N,K", [(16, 128), (48, 640), (272, 512), (300, 1024), (4096, 16384), (12288, 4096)])
def test_pack_fp4_matches_oracle(N, K):
    _announce("pack_fp4 N=%d K=%d" % (N, K))
    rng = np.random.default_rng(N + K)
    W = workloads.w_latent(rng, N, K)
    Wp, _ = hbl.hbl_quantize_weights(to_dev(W))
    W4 = hbl.hbl_pack_fp4(Wp, K)
    _sync()
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    assert np.array_equal(to_host(W4).reshape(-1), fp4_library_order(oracle.pack_fp4(Wq)))


FP4_CASES = [
    # (M, K, N, hadamard, x dtype, y dtype, norm)
    (1, 512, 64, True, "f32", "f32", hbl.HBL_NORM_RMS),
    (37, 1024, 272, True, "bf16", "bf16", hbl.HBL_NORM_LN),
    (300, 2048, 4096, False, "bf16", "bf16", hbl.HBL_NORM_RMS),
    (4100, 4096, 8000, True, "f32", "bf16", hbl.HBL_NORM_NONE),
    (513, 32768, 256, True, "bf16", "f32", hbl.HBL_NORM_RMS),
    (8192, 16384, 4096, True, "bf16", "bf16", hbl.HBL_NORM_RMS),   # the 7B / 3B Wdown shape
    (8192, 4096, 32768, False, "bf16", "bf16", hbl.HBL_NORM_RMS),  # the 3B gate/up shape
]


@pytest.mark.parametrize("M,K,N,had,xdt,ydt,norm", FP4_CASES)
def test_forward_fp4_matches_int8_path_and_oracle(M, K, N, had, xdt, ydt, norm):
    import torch
    _announce("forward_fp4 M=%d K=%d N=%d had=%d %s->%s norm=%d" % (M, K, N, had, xdt, ydt, norm))
    rng = np.random.default_rng(M * 7 + K + N)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(2.0)).astype(np.float32)
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    cfg = hbl.Config(act_bits=4, hadamard=had, norm=norm)
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    W4 = hbl.hbl_pack_fp4(Wp, K)
    Y4 = hbl.hbl_forward_fp4(Xd, W4, alpha, N, cfg, y_dtype=yt)
    small = torch.empty(hbl.hbl_workspace_bytes(M, K, cfg), dtype=torch.uint8, device="cuda:0")
    Y8 = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt, ws=small)
    c6, xs6 = hbl.hbl_quantize_activations_fp6(Xd, cfg)
    Ys = hbl.hbl_gemm_fp6fp4(c6, xs6, K, W4, alpha, N, y_dtype=yt)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    _sync()
    got = to_host(Y4)
    assert np.array_equal(got, to_host(Y8))
    assert np.array_equal(got, to_host(Ys))
    assert np.array_equal(to_host(xs6), to_host(xs))
    rows = workloads.sample_rows(M, 16)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 16)]))
    q = unpack_codes(to_host(codes)[rows], K, 4)
    a = to_host(alpha)[0]
    y_exact = oracle.rescale(oracle.int_gemm(q, oracle.ternarize(W[cols], a, 1e-5)), to_host(xs)[rows], a)
    sub = got[np.ix_(rows, cols)]
    assert np.array_equal(sub, y_exact if ydt == "f32" else oracle.f32_to_bf16(y_exact))


def test_forward_fp4_empty_and_deterministic():
    import torch
    _announce("forward_fp4 empty / deterministic")
    cfg = hbl.Config(act_bits=4)
    rng = np.random.default_rng(5)
    W = workloads.w_latent(rng, 512, 2048)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    W4 = hbl.hbl_pack_fp4(Wp, 2048)
    X = to_dev(workloads.f32_to_bf16_bits(workloads.x_outlier_gaussian(rng, 700, 2048, 4, 30.0)[0]))
    Y1 = hbl.hbl_forward_fp4(X, W4, alpha, 512, cfg)
    Y2 = hbl.hbl_forward_fp4(X, W4, alpha, 512, cfg)
    E = hbl.hbl_forward_fp4(torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda:0"), W4, alpha, 512, cfg)
    _sync()
    assert np.array_equal(to_host(Y1), to_host(Y2)) and E.shape == (0, 512)
