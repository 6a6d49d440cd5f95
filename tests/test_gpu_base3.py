"""GPU parity of the base-3 weight path (five ternary weights per byte)
through the C ABI: packing bit for bit against the oracle's O13, the GEMV's
int32 sums and rescale bit for bit against the oracle's O9/O10, and the
forward bit for bit against hbl_forward on the same ternary values."""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import check_codes_end_to_end, check_y, to_dev, to_host, unpack_codes, y_to_f32

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _announce(msg):
    print("[case] " + msg, flush=True)


def _random_codes(rng, M, K, bits):
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    q = rng.integers(lo, hi + 1, size=(M, K)).astype(np.int8)
    return q, (q if bits == 8 else oracle.pack_int4(q))


@pytest.mark.parametrize("N,K", [(1, 16), (16, 80), (48, 96), (7, 1008), (300, 4000), (4096, 8192), (64, 16384),
                                 (5, 32768)])
def test_pack_base3_parity(N, K):
    _announce("pack base3 N=%d K=%d" % (N, K))
    rng = np.random.default_rng(N + K)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    W3 = hbl.hbl_pack_base3(to_dev(oracle.pack_ternary(Wq)), K)
    _sync()
    assert np.array_equal(to_host(W3), oracle.pack_base3(Wq))


GEMV_CASES = [
    # (M, K, N, bits): every M, one- to four-wave blocks, ragged N and K not a multiple of 80
    (1, 16, 1, 8), (2, 80, 7, 4), (3, 1008, 33, 8), (4, 1024, 16, 4), (1, 4000, 100, 4), (2, 4096, 64, 8),
    (3, 5120, 24, 4), (4, 8192, 40, 8), (1, 8192, 4096, 4), (1, 8192, 4096, 8), (2, 16384, 72, 4),
    (4, 16384, 1000, 8), (1, 10240, 9, 8), (3, 15360, 8, 4),
]


@pytest.mark.parametrize("M,K,N,bits", GEMV_CASES)
def test_gemm_base3_int32_sums_exact(M, K, N, bits):
    """xscale = 1 and alpha = 1 make the fp32 output the int32 sum itself."""
    _announce("gemm base3 M=%d K=%d N=%d a%d" % (M, K, N, bits))
    import torch
    rng = np.random.default_rng(M * 17 + K + N * 3 + bits)
    q, packed = _random_codes(rng, M, K, bits)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    ones = torch.ones(M, dtype=torch.float32, device="cuda:0")
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    Y = hbl.hbl_gemm_base3(to_dev(packed), ones, bits, K, to_dev(oracle.pack_base3(Wq)), one, N)
    _sync()
    assert np.array_equal(to_host(Y), oracle.int_gemm(q, Wq).astype(np.float32))


@pytest.mark.parametrize("M,K,bits", [(4, 16384, 8), (3, 16384, 4), (1, 8000, 8)])
def test_gemm_base3_extreme_sums(M, K, bits):
    """Every code at an end of its range against all -1 (or +1) weights."""
    _announce("gemm base3 extremes M=%d K=%d a%d" % (M, K, bits))
    import torch
    N = 24
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    q = np.full((M, K), lo, dtype=np.int8)
    q[1::2] = hi
    Wq = -np.ones((N, K), dtype=np.int8)
    Wq[N // 2:] = 1
    ones = torch.ones(M, dtype=torch.float32, device="cuda:0")
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    Y = hbl.hbl_gemm_base3(to_dev(q if bits == 8 else oracle.pack_int4(q)), ones, bits, K,
                           to_dev(oracle.pack_base3(Wq)), one, N)
    _sync()
    acc = oracle.int_gemm(q, Wq)
    assert np.abs(acc).max() == -lo * K
    assert np.array_equal(to_host(Y), acc.astype(np.float32))


@pytest.mark.parametrize("M,bits,ydt", [(1, 8, "f32"), (2, 4, "bf16"), (3, 8, "bf16"), (4, 4, "f32")])
def test_gemm_base3_rescale_exact(M, bits, ydt):
    import torch
    K, N = 2048, 136
    rng = np.random.default_rng(M + bits + 7)
    q, packed = _random_codes(rng, M, K, bits)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) * np.float32(0.01)).astype(np.float32)
    alpha = np.array([0.0173], np.float32)
    Y = hbl.hbl_gemm_base3(to_dev(packed), to_dev(d), bits, K, to_dev(oracle.pack_base3(Wq)), to_dev(alpha), N,
                           y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    _sync()
    y_ref = oracle.rescale(oracle.int_gemm(q, Wq), d, alpha[0])
    assert np.array_equal(to_host(Y), y_ref if ydt == "f32" else oracle.f32_to_bf16(y_ref))


@pytest.mark.parametrize("M,K,N,bits", [(1, 8192, 4096, 4), (4, 4096, 2048, 8), (2, 16384, 512, 4)])
def test_gemm_base3_equals_2bit_gemm(M, K, N, bits):
    """The same ternary values in either storage give the same output bits."""
    import torch
    rng = np.random.default_rng(M + K + N)
    q, packed = _random_codes(rng, M, K, bits)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) + np.float32(0.5)).astype(np.float32)
    alpha = np.array([0.031], np.float32)
    Wp = to_dev(oracle.pack_ternary(Wq))
    W3 = hbl.hbl_pack_base3(Wp, K)
    Y2 = hbl.hbl_gemm(to_dev(packed), to_dev(d), bits, K, Wp, to_dev(alpha), N, y_dtype=torch.bfloat16)
    Y3 = hbl.hbl_gemm_base3(to_dev(packed), to_dev(d), bits, K, W3, to_dev(alpha), N, y_dtype=torch.bfloat16)
    _sync()
    assert np.array_equal(to_host(Y2), to_host(Y3))


@pytest.mark.parametrize("M", [1, 2, 4])
def test_forward_base3_decode_layer(M):
    """The decode layer (K = 8192, N = 4096, INT4, fp32 in, bf16 out) with the
    weights in base-3 storage: bit for bit hbl_forward with the 2-bit weights,
    and against the oracle's own pipeline (a code may flip at a rounding
    boundary, checked; those rows use the oracle's arithmetic on the GPU's code)."""
    import torch
    layer = workloads.DECODE[0]
    K, N, bits = layer.K, layer.N, layer.act_bits
    _announce("forward base3 decode M=%d K=%d N=%d a%d" % (M, K, N, bits))
    rng = np.random.default_rng(11 + M)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    W = workloads.w_latent(rng, N, K)
    Wq, _, a_ref = oracle.quantize_weights(W)
    alpha = to_dev(np.array([a_ref], np.float32))
    Wp = to_dev(oracle.pack_ternary(Wq))
    W3 = to_dev(oracle.pack_base3(Wq))
    cfg = hbl.Config(act_bits=bits, hadamard=layer.hadamard)
    Xd = to_dev(X)
    Y3 = hbl.hbl_forward_base3(Xd, W3, alpha, N, cfg, y_dtype=torch.bfloat16)
    Y2 = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=torch.bfloat16)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    _sync()
    assert np.array_equal(to_host(Y3), to_host(Y2))
    ref = oracle.quantize_activations(X, bits=bits, hadamard=layer.hadamard)
    q_gpu = unpack_codes(to_host(codes), K, bits)
    check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], "base3 forward codes")
    y_exact = oracle.rescale(oracle.int_gemm(q_gpu, Wq), to_host(xs), a_ref)
    assert np.array_equal(to_host(Y3), oracle.f32_to_bf16(y_exact))
    flipped = np.any(q_gpu != ref["q"], axis=1)
    q_cmp = np.where(flipped[:, None], q_gpu, ref["q"])
    check_y(y_to_f32(to_host(Y3)), oracle.rescale(oracle.int_gemm(q_cmp, Wq), ref["d"], a_ref), "base3 y",
            bf16_out=True)


@pytest.mark.parametrize("bits,norm,use_gain,xdt,had", [(8, hbl.HBL_NORM_LN, True, "bf16", True),
                                                        (4, hbl.HBL_NORM_NONE, True, "f32", False),
                                                        (8, hbl.HBL_NORM_RMS, False, "bf16", False)])
def test_forward_base3_configs(bits, norm, use_gain, xdt, had):
    """Norms, gain, bf16 input, INT8 and the plain layer: bit for bit hbl_forward."""
    import torch
    M, K, N = 3, 4096, 528
    _announce("forward base3 a%d norm=%d gain=%d %s had=%d" % (bits, norm, use_gain, xdt, had))
    rng = np.random.default_rng(bits + norm * 3 + use_gain)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    Xh = workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X
    W = workloads.w_latent(rng, N, K)
    Wq, _, a_ref = oracle.quantize_weights(W)
    gain = to_dev((rng.standard_normal(K) * 0.5 + 1.0).astype(np.float32)) if use_gain else None
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm)
    Xd = to_dev(Xh)
    alpha = to_dev(np.array([a_ref], np.float32))
    Y3 = hbl.hbl_forward_base3(Xd, to_dev(oracle.pack_base3(Wq)), alpha, N, cfg, y_dtype=torch.float32, gain=gain)
    Y2 = hbl.hbl_forward(Xd, to_dev(oracle.pack_ternary(Wq)), alpha, N, cfg, y_dtype=torch.float32, gain=gain)
    _sync()
    assert np.array_equal(to_host(Y3), to_host(Y2))
