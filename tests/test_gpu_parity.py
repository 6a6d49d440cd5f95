"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Small cases compare every element; the full-size layer workloads compare a
sample of 64 rows (first, last, evenly spaced) that the oracle can compute,
in the same launch configuration the benchmark times (hbl_quantize_weights,
then hbl_forward).  Tolerances: see tests/parity.py.
"""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import (check_codes_end_to_end, check_codes_given_inputs, check_dw, check_y, check_z, to_dev, to_host,
                    unpack_codes, y_to_f32)

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _announce(msg):
    print("[case] " + msg, flush=True)


# ================================================================= weights ==
@pytest.mark.parametrize("N,K,dt", [(256, 256, "f32"), (48, 80, "f32"), (2048, 2048, "f32"), (96, 4096, "bf16"),
                                    (4096, 16384, "bf16")])
def test_quantize_weights_parity(N, K, dt):
    _announce("weights N=%d K=%d %s" % (N, K, dt))
    rng = np.random.default_rng(N * 7 + K)
    W = workloads.w_latent(rng, N, K)
    if dt == "bf16":
        W = workloads.f32_to_bf16_bits(W)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W), eps=1e-5)
    _sync()
    Wp, a_gpu = to_host(Wp), to_host(alpha)[0]
    a_ref = oracle.weight_alpha(W)
    assert abs(float(a_gpu) - float(a_ref)) <= 1e-6 * float(a_ref)
    # bit-exact packing given the GPU's alpha
    Wq = oracle.ternarize(W, a_gpu, 1e-5)
    assert np.array_equal(Wp, oracle.pack_ternary(Wq))


def test_quantize_weights_hand_cases(golden):
    g = golden("ternary_hand.txt")
    for key in ("tie", "mean", "eps"):
        W = np.tile(np.array(g[key + "_latent"], np.float32), 4)[None, :]      # mean|W| unchanged by tiling
        Wp, alpha = hbl.hbl_quantize_weights(to_dev(W), eps=g[key + "_eps"])
        _sync()
        q = oracle.unpack_ternary(to_host(Wp), 16)[0]
        assert q.tolist() == g[key + "_ternary"] * 4, key
    gp = golden("pack_ternary_k16.txt")
    W = np.array([gp["ternary"]], np.float32) * np.float32(0.75)   # alpha = 0.75*mean|t|; |W|/alpha >= 1.45 or 0
    Wp, _ = hbl.hbl_quantize_weights(to_dev(W), eps=0.0)
    _sync()
    assert to_host(Wp)[0].tolist() == gp["bytes"]
    Wz = np.zeros((16, 64), np.float32)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(Wz), eps=0.0)
    _sync()
    assert to_host(alpha)[0] == 0.0 and not to_host(Wp).any()


# ============================================================= activations ==
ACT_CASES = [
    # (K, x_dtype, bits, hadamard, norm, a4_mode, gain, M)
    (256, "f32", 8, True, hbl.HBL_NORM_RMS, 0, False, 8),
    (256, "bf16", 4, True, hbl.HBL_NORM_RMS, 0, False, 37),
    (512, "f32", 4, True, hbl.HBL_NORM_LN, 1, True, 5),
    (1024, "bf16", 8, False, hbl.HBL_NORM_RMS, 0, True, 9),
    (2048, "bf16", 8, True, hbl.HBL_NORM_RMS, 0, False, 33),
    (2048, "f32", 4, True, hbl.HBL_NORM_NONE, 0, False, 7),
    (4096, "bf16", 4, False, hbl.HBL_NORM_RMS, 0, False, 11),
    (8192, "f32", 4, True, hbl.HBL_NORM_RMS, 0, False, 16),
    (16384, "bf16", 4, True, hbl.HBL_NORM_RMS, 0, False, 6),
    (16384, "bf16", 8, True, hbl.HBL_NORM_LN, 0, True, 3),
    (32768, "f32", 8, True, hbl.HBL_NORM_RMS, 0, False, 2),
    (32768, "bf16", 4, True, hbl.HBL_NORM_RMS, 1, False, 2),
    # LayerNorm without a gain (Hadamard path folds the mean into element 0), plain LN, NONE with a gain
    (2048, "bf16", 4, True, hbl.HBL_NORM_LN, 0, False, 9),
    (16384, "f32", 8, True, hbl.HBL_NORM_LN, 0, False, 3),
    (4096, "f32", 8, False, hbl.HBL_NORM_LN, 0, False, 5),
    (1024, "bf16", 8, True, hbl.HBL_NORM_NONE, 0, True, 4),
    (256, "f32", 8, False, hbl.HBL_NORM_RMS, 0, False, 3),
]


@pytest.mark.parametrize("K,dt,bits,had,norm,a4,use_gain,M", ACT_CASES)
def test_quantize_activations_parity(K, dt, bits, had, norm, a4, use_gain, M):
    _announce("act K=%d %s a%d H=%d norm=%d a4=%d gain=%d M=%d" % (K, dt, bits, had, norm, a4, use_gain, M))
    rng = np.random.default_rng(K + bits + M)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(3.0)).astype(np.float32)  # nonzero mean
    if M > 2:
        X[1] = 0.0                                   # an all-zero row
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if use_gain else None
    Xh = workloads.f32_to_bf16_bits(X) if dt == "bf16" else X
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm, a4_mode=a4)
    codes, xs, z, s = hbl.hbl_quantize_activations(to_dev(Xh), cfg, gain=None if gain is None else to_dev(gain),
                                                   z_debug=True, s_debug=True)
    _sync()
    q_gpu = unpack_codes(to_host(codes), K, bits)
    z_gpu, d_gpu, s_gpu = to_host(z), to_host(xs), to_host(s)
    ref = oracle.quantize_activations(Xh, bits=bits, hadamard=had, gain=gain, norm=norm, a4_mode=a4)
    check_z(z_gpu, ref["z"], "z")
    check_codes_given_inputs(z_gpu, s_gpu, d_gpu, q_gpu, bits, a4, 1e-5, "codes")
    n_boundary = check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], "end-to-end codes")
    assert n_boundary <= max(2, q_gpu.size // 10000)
    if M > 2:
        assert not q_gpu[1].any() and d_gpu[1] == 0.0


def test_quantize_activations_deterministic():
    rng = np.random.default_rng(5)
    X, _ = workloads.x_laplace_mixture(rng, 64, 4096)
    Xd = to_dev(workloads.f32_to_bf16_bits(X))
    outs = []
    for _ in range(2):
        c, xs, z, _ = hbl.hbl_quantize_activations(Xd, hbl.Config(act_bits=4), z_debug=True)
        _sync()
        outs.append((to_host(c), to_host(xs), to_host(z)))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a, b)


# ===================================================================== GEMM ==
def _random_codes(rng, M, K, bits):
    q = rng.integers(-128 if bits == 8 else -8, 128 if bits == 8 else 8, size=(M, K)).astype(np.int8)
    packed = q if bits == 8 else oracle.pack_int4(q)
    return q, packed


GEMM_CASES = [
    # (M, K, N, bits) -- prefill tiles 128 x 128 or 128 x 256, decode (M <= 64) tiles 16 columns
    (300, 2048, 272, 8), (300, 2048, 272, 4), (129, 256, 16, 8), (128, 1024, 128, 4), (257, 128, 400, 8), (1024, 4096, 1024, 8), (520, 16384, 384, 4),
    (1, 8192, 4096, 4), (7, 8192, 512, 8), (16, 4096, 1024, 4), (17, 2048, 256, 4), (33, 1024, 64, 8),
    (64, 8192, 1024, 4), (65, 512, 192, 4), (64, 128, 32, 8),
    # 17..64 tokens, K <= 8192, N >= 8192: 32 columns per decode block (N not a multiple of 32 too)
    (40, 4096, 8208, 8), (20, 8192, 8192, 4), (64, 256, 8240, 4), (33, 2048, 16384, 8), (17, 16384, 64, 8),
    # M <= 4 with K a power of two in [1024, 16384]: the vector-ALU GEMV, every K and M
    (1, 1024, 48, 8), (2, 2048, 64, 4), (3, 4096, 32, 8), (4, 8192, 16, 8), (4, 16384, 80, 4), (1, 16384, 4096, 8),
    (2, 1024, 32, 4), (3, 8192, 64, 4), (1, 4096, 1024, 4), (2, 512, 64, 8), (3, 32768, 32, 4),
    # >= 512 tiles of 128 x 256: the large-tile kernel, ragged in M and N
    (4100, 256, 4000, 4), (4100, 384, 4000, 8),
    # the largest K (accumulators up to 2^28 before the shift back)
    (200, 32768, 256, 8), (130, 32768, 272, 4),
]


@pytest.mark.parametrize("M,K,N,bits", GEMM_CASES)
def test_gemm_int32_accumulators_exact(M, K, N, bits):
    """xscale = 1 and alpha = 1 make the fp32 output the int32 accumulator itself."""
    _announce("gemm M=%d K=%d N=%d a%d" % (M, K, N, bits))
    import torch
    rng = np.random.default_rng(M * 131 + K + N + bits)
    q, packed = _random_codes(rng, M, K, bits)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Wp = oracle.pack_ternary(Wq)
    ones = torch.ones(M, dtype=torch.float32, device="cuda:0")
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    Y = hbl.hbl_gemm(to_dev(packed), ones, bits, K, to_dev(Wp), one, N)
    _sync()
    acc = oracle.int_gemm(q, Wq)
    assert np.array_equal(to_host(Y), acc.astype(np.float32))


@pytest.mark.parametrize("M,K,bits", [(130, 32768, 8), (130, 32768, 4), (20, 32768, 8), (3, 16384, 4), (1, 16384, 8)])
def test_gemm_extreme_accumulators(M, K, bits):
    """Largest |acc| the formats allow: every code at the negative end of its
    range against all -1 weights (and the positive end in alternate rows)."""
    _announce("gemm extremes M=%d K=%d a%d" % (M, K, bits))
    N = 64
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    q = np.full((M, K), lo, dtype=np.int8)
    q[1::2] = hi
    packed = q if bits == 8 else oracle.pack_int4(q)
    Wq = -np.ones((N, K), dtype=np.int8)
    Wq[:, : K // 2][N // 2:] = 1
    import torch
    ones = torch.ones(M, dtype=torch.float32, device="cuda:0")
    one = torch.ones(1, dtype=torch.float32, device="cuda:0")
    Y = hbl.hbl_gemm(to_dev(packed), ones, bits, K, to_dev(oracle.pack_ternary(Wq)), one, N)
    _sync()
    acc = oracle.int_gemm(q, Wq)
    assert np.abs(acc).max() == -lo * K
    assert np.array_equal(to_host(Y), acc.astype(np.float32))


@pytest.mark.parametrize("M,bits,ydt", [(200, 8, "f32"), (200, 4, "bf16"), (5, 4, "f32"), (40, 8, "bf16"),
                                        (1, 8, "f32"), (3, 4, "bf16")])
def test_gemm_rescale_epilogue_exact(M, bits, ydt):
    import torch
    K, N = 1024, 256
    rng = np.random.default_rng(M + bits)
    q, packed = _random_codes(rng, M, K, bits)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) * np.float32(0.01)).astype(np.float32)
    alpha = np.array([0.0173], np.float32)
    Y = hbl.hbl_gemm(to_dev(packed), to_dev(d), bits, K, to_dev(oracle.pack_ternary(Wq)), to_dev(alpha), N,
                     y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    _sync()
    y_ref = oracle.rescale(oracle.int_gemm(q, Wq), d, alpha[0])
    if ydt == "f32":
        assert np.array_equal(to_host(Y), y_ref)
    else:
        assert np.array_equal(to_host(Y), oracle.f32_to_bf16(y_ref))


# ================================================================= forward ==
def _run_layer(layer, rows, seed=0):
    """Quantise weights and run hbl_forward on the full layer (as the bench
    does), plus the stage entry points for z/s; return host arrays for `rows`."""
    import torch
    X, W, _ = workloads.make_inputs(layer, seed)
    Xd, Wd = to_dev(X), to_dev(W)
    cfg = hbl.Config(act_bits=layer.act_bits, hadamard=layer.hadamard)
    Wp, alpha = hbl.hbl_quantize_weights(Wd, eps=1e-5)
    ydt = torch.float32 if layer.y_dtype == "f32" else torch.bfloat16
    Y = hbl.hbl_forward(Xd, Wp, alpha, layer.N, cfg, y_dtype=ydt)
    codes, xs, z, s = hbl.hbl_quantize_activations(Xd, cfg, z_debug=True, s_debug=True)
    ridx = torch.from_numpy(rows).to("cuda:0")
    out = {
        "Y": to_host(Y.index_select(0, ridx)),
        "codes": to_host(codes.index_select(0, ridx)),
        "xs": to_host(xs.index_select(0, ridx)),
        "z": to_host(z.index_select(0, ridx)),
        "s": to_host(s.index_select(0, ridx)),
        "Wp": to_host(Wp),
        "alpha": to_host(alpha)[0],
    }
    # the stage entry points and hbl_forward must agree bit for bit
    Y2 = hbl.hbl_gemm(codes, xs, layer.act_bits, layer.K, Wp, alpha, layer.N, y_dtype=ydt)
    _sync()
    assert np.array_equal(to_host(Y2.index_select(0, ridx)), out["Y"])
    del Xd, Wd, Y, Y2, codes, z
    torch.cuda.empty_cache()
    Xs = X[rows]
    return Xs, W, out


def _check_layer(layer, rows):
    _announce("layer %s rows=%d" % (layer.desc, len(rows)))
    Xs, W, g = _run_layer(layer, rows)
    K, bits = layer.K, layer.act_bits
    a_ref = oracle.weight_alpha(W)
    assert abs(float(g["alpha"]) - float(a_ref)) <= 1e-6 * float(a_ref)
    Wq = oracle.ternarize(W, g["alpha"], 1e-5)
    assert np.array_equal(g["Wp"], oracle.pack_ternary(Wq))
    ref = oracle.quantize_activations(Xs, bits=bits, hadamard=layer.hadamard)
    q_gpu = unpack_codes(g["codes"], K, bits)
    check_z(g["z"], ref["z"], layer.name + " z")
    check_codes_given_inputs(g["z"], g["s"], g["xs"], q_gpu, bits, 0, 1e-5, layer.name + " codes")
    nb = check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], layer.name + " end-to-end codes")
    # int32 accumulators: the oracle's GEMM on the GPU's own codes and weights, then the
    # oracle's rescale with the GPU's own scales reproduces the fp32 output exactly
    acc = oracle.int_gemm(q_gpu, Wq)
    y_exact = oracle.rescale(acc, g["xs"], g["alpha"])
    if layer.y_dtype == "f32":
        assert np.array_equal(g["Y"], y_exact)
    else:
        assert np.array_equal(g["Y"], oracle.f32_to_bf16(y_exact))
    # end to end against the oracle's own pipeline.  Rows where a code flipped at a
    # rounding boundary (allowed above) are compared with the oracle's arithmetic on
    # those codes; every other row with the oracle's own codes.
    flipped = np.any(q_gpu != ref["q"], axis=1)
    q_cmp = np.where(flipped[:, None], q_gpu, ref["q"])
    y_ref = oracle.rescale(oracle.int_gemm(q_cmp, Wq), ref["d"], a_ref)
    check_y(y_to_f32(g["Y"]), y_ref, layer.name + " y", bf16_out=layer.y_dtype == "bf16")
    print("[parity] %s: %d boundary code flips in %d of %d rows" % (layer.name, nb, int(flipped.sum()), len(rows)))
    return nb


def test_forward_small_layer_all_rows():
    layer = workloads.SMALL
    _check_layer(layer, np.arange(layer.M))


def test_forward_wo_1p3b_sampled():
    layer = workloads.WO_1P3B
    _check_layer(layer, workloads.sample_rows(layer.M))


def test_forward_wdown_7b_sampled():
    layer = workloads.WDOWN_7B
    _check_layer(layer, workloads.sample_rows(layer.M, 48))


@pytest.mark.parametrize("layer", workloads.DECODE, ids=lambda l: l.name)
def test_forward_decode_all_rows(layer):
    _check_layer(layer, np.arange(layer.M))


@pytest.mark.parametrize("layer", workloads.CHAIN_3B, ids=lambda l: l.name)
def test_forward_chain_3b_sampled(layer):
    _check_layer(layer, workloads.sample_rows(layer.M, 32))


# One token and K a power of two in [1024, 16384]: hbl_forward runs as one fused
# launch (each block quantises the row itself).  It must equal the two stage
# entry points bit for bit, for every K, width, norm and dtype it serves (and
# the few-token shapes next to it, which take the two stage kernels).
SMALL_M_CASES = [
    # (M, K, N, bits, hadamard, x dtype, y dtype, norm, gain)
    (1, 8192, 4096, 4, True, "f32", "bf16", hbl.HBL_NORM_RMS, False),
    (1, 1024, 64, 8, True, "bf16", "f32", hbl.HBL_NORM_RMS, False),
    (1, 2048, 128, 4, True, "f32", "f32", hbl.HBL_NORM_LN, False),
    (1, 4096, 256, 8, False, "bf16", "bf16", hbl.HBL_NORM_RMS, True),
    (1, 16384, 96, 4, True, "bf16", "bf16", hbl.HBL_NORM_LN, True),
    (1, 8192, 512, 8, True, "f32", "f32", hbl.HBL_NORM_NONE, False),
    (1, 16384, 32, 8, False, "f32", "bf16", hbl.HBL_NORM_RMS, False),
    (1, 1024, 48, 4, False, "f32", "f32", hbl.HBL_NORM_LN, False),
    (1, 4096, 64, 4, True, "bf16", "f32", hbl.HBL_NORM_RMS, True),
    (2, 2048, 128, 4, True, "f32", "f32", hbl.HBL_NORM_LN, False),
    (4, 8192, 512, 8, True, "f32", "bf16", hbl.HBL_NORM_RMS, False),
]


@pytest.mark.parametrize("M,K,N,bits,had,xdt,ydt,norm,use_gain", SMALL_M_CASES)
def test_forward_small_m_matches_stages(M, K, N, bits, had, xdt, ydt, norm, use_gain):
    import torch
    _announce("forward small M=%d K=%d N=%d a%d had=%d %s->%s norm=%d gain=%d" % (M, K, N, bits, had, xdt, ydt,
                                                                                norm, use_gain))
    rng = np.random.default_rng(M * 7 + K + N + bits)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(2.0)).astype(np.float32)
    W = workloads.w_latent(rng, N, K)
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if use_gain else None
    Xh = workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X
    Xd = to_dev(Xh)
    gd = None if gain is None else to_dev(gain)
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    Y = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt, gain=gd)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg, gain=gd)
    Y2 = hbl.hbl_gemm(codes, xs, bits, K, Wp, alpha, N, y_dtype=yt)
    _sync()
    assert np.array_equal(to_host(Y), to_host(Y2))
    # and against the oracle's arithmetic on those codes and scales
    q = unpack_codes(to_host(codes), K, bits)
    Wq = oracle.ternarize(W, to_host(alpha)[0], 1e-5)
    y_exact = oracle.rescale(oracle.int_gemm(q, Wq), to_host(xs), to_host(alpha)[0])
    got = to_host(Y)
    assert np.array_equal(got, y_exact if ydt == "f32" else oracle.f32_to_bf16(y_exact))


# Up to 64 tokens (outside the one-token fused shapes) the decode GEMM reads
# the codes that hbl_forward keeps in its tiled order; the result must equal
# the stage entry points (row-major codes) bit for bit, and the oracle's
# arithmetic on sampled columns.  Covers one and several 16-row tiles, partial
# last tiles, 32-column blocks (17-64 tokens, N >= 8192, K <= 8192), K from
# one super-step (256) to the maximum (32768), and few-token shapes the GEMV
# does not serve (K below 1024 or above 16384).
DECODE_TILED_CASES = [
    # (M, K, N, bits, hadamard, x dtype, y dtype)
    (5, 4096, 1024, 8, True, "f32", "f32"),
    (16, 8192, 4096, 4, True, "bf16", "bf16"),
    (17, 2048, 8192, 8, True, "f32", "bf16"),
    (33, 8192, 8192, 4, True, "bf16", "f32"),
    (64, 32768, 512, 8, True, "f32", "f32"),
    (64, 256, 16384, 4, False, "f32", "bf16"),
    (48, 1024, 2048, 4, True, "bf16", "bf16"),
    (2, 512, 64, 4, True, "f32", "f32"),
    (4, 32768, 64, 8, False, "bf16", "f32"),
    (31, 16384, 1024, 8, True, "bf16", "bf16"),
]


@pytest.mark.parametrize("M,K,N,bits,had,xdt,ydt", DECODE_TILED_CASES)
def test_forward_decode_tiled_matches_stages(M, K, N, bits, had, xdt, ydt):
    import torch
    _announce("forward decode-tiled M=%d K=%d N=%d a%d had=%d %s->%s" % (M, K, N, bits, had, xdt, ydt))
    rng = np.random.default_rng(M * 13 + K + N + bits)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    cfg = hbl.Config(act_bits=bits, hadamard=had)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    Y = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    Y2 = hbl.hbl_gemm(codes, xs, bits, K, Wp, alpha, N, y_dtype=yt)
    _sync()
    got = to_host(Y)
    assert np.array_equal(got, to_host(Y2))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 40)]))
    q = unpack_codes(to_host(codes), K, bits)
    a = to_host(alpha)[0]
    y_exact = oracle.rescale(oracle.int_gemm(q, oracle.ternarize(W[cols], a, 1e-5)), to_host(xs), a)
    assert np.array_equal(got[:, cols], y_exact if ydt == "f32" else oracle.f32_to_bf16(y_exact))


# INT4 prefill shapes with the larger workspace (hbl_forward_workspace_bytes)
# run on the FP6 x FP4 matrix cores: codes as FP6 E3M2, weights as FP4 E2M1,
# exact fp32 sums.  Y must equal the INT8-MFMA path (the smaller workspace)
# and the stage entry points bit for bit, and the oracle's arithmetic on
# sampled columns.  Ragged M and N, K from 512 to the maximum, both norms,
# with and without the Hadamard, both input and output dtypes.
F6F4_CASES = [
    # (M, K, N, hadamard, x dtype, y dtype, norm)
    (300, 2048, 32768, True, "bf16", "bf16", hbl.HBL_NORM_RMS),
    (4100, 512, 8000, True, "f32", "f32", hbl.HBL_NORM_RMS),
    (1024, 4096, 8192, False, "bf16", "bf16", hbl.HBL_NORM_RMS),
    (4096, 32768, 2048, True, "bf16", "f32", hbl.HBL_NORM_LN),
    (8192, 16384, 4096, True, "bf16", "bf16", hbl.HBL_NORM_RMS),
]


@pytest.mark.parametrize("M,K,N,had,xdt,ydt,norm", F6F4_CASES)
def test_forward_f6f4_matches_int8_path(M, K, N, had, xdt, ydt, norm):
    import torch
    _announce("forward fp6xfp4 M=%d K=%d N=%d had=%d %s->%s norm=%d" % (M, K, N, had, xdt, ydt, norm))
    rng = np.random.default_rng(M + K * 3 + N)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(2.0)).astype(np.float32)
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    cfg = hbl.Config(act_bits=4, hadamard=had, norm=norm)
    small = hbl.hbl_workspace_bytes(M, K, cfg)
    big = hbl.hbl_forward_workspace_bytes(M, K, N, cfg)
    assert big > small  # the shape takes the FP6 x FP4 path with the larger workspace
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    Y6 = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt,
                         ws=torch.empty(big, dtype=torch.uint8, device="cuda:0"))
    Y8 = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt,
                         ws=torch.empty(small, dtype=torch.uint8, device="cuda:0"))
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    Y2 = hbl.hbl_gemm(codes, xs, 4, K, Wp, alpha, N, y_dtype=yt)
    _sync()
    got = to_host(Y6)
    assert np.array_equal(got, to_host(Y8))
    assert np.array_equal(got, to_host(Y2))
    rows = workloads.sample_rows(M, 24)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 24)]))
    q = unpack_codes(to_host(codes)[rows], K, 4)
    a = to_host(alpha)[0]
    y_exact = oracle.rescale(oracle.int_gemm(q, oracle.ternarize(W[cols], a, 1e-5)), to_host(xs)[rows], a)
    sub = got[np.ix_(rows, cols)]
    assert np.array_equal(sub, y_exact if ydt == "f32" else oracle.f32_to_bf16(y_exact))


@pytest.mark.parametrize("M,K,N,xdt,wdt", [(4096, 2048, 4096, "bf16", "f32"), (2048, 8192, 8192, "f32", "bf16")])
def test_forward_latent_f6f4_matches_two_calls(M, K, N, xdt, wdt):
    """Latent weights with the larger workspace: activation codes as FP6 (in
    the shared activation / packing grid for K <= 2048), weights packed, then
    converted to FP4; equal to hbl_quantize_weights + hbl_forward (INT8 path)."""
    import torch
    _announce("forward_latent fp6xfp4 M=%d K=%d N=%d x %s W %s" % (M, K, N, xdt, wdt))
    rng = np.random.default_rng(M + K + N + 4)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    Wd = to_dev(workloads.f32_to_bf16_bits(W) if wdt == "bf16" else W)
    cfg = hbl.Config(act_bits=4, hadamard=True)
    big = hbl.hbl_forward_workspace_bytes(M, K, N, cfg)
    assert big > hbl.hbl_workspace_bytes(M, K, cfg)
    Y, Wp, alpha = hbl.hbl_forward_latent(Xd, Wd, cfg, eps=1e-5, y_dtype=torch.bfloat16,
                                          ws=torch.empty(big, dtype=torch.uint8, device="cuda:0"))
    Wp2, alpha2 = hbl.hbl_quantize_weights(Wd, eps=1e-5)
    small = torch.empty(hbl.hbl_workspace_bytes(M, K, cfg), dtype=torch.uint8, device="cuda:0")
    Y2 = hbl.hbl_forward(Xd, Wp2, alpha2, N, cfg, y_dtype=torch.bfloat16, ws=small)
    _sync()
    assert np.array_equal(to_host(alpha), to_host(alpha2))
    assert np.array_equal(to_host(Wp), to_host(Wp2))
    assert np.array_equal(to_host(Y), to_host(Y2))


# hbl_forward_latent: weights ternarised and the forward run in three launches
# (activation quantisation and weight packing share a grid); Y, W_packed and
# alpha must equal hbl_quantize_weights + hbl_forward bit for bit.
LATENT_CASES = [
    # (M, K, N, bits, hadamard, x dtype, W dtype, y dtype)
    (4096, 2048, 2048, 8, True, "bf16", "f32", "bf16"),   # the 1.3B Wo shape: shared grid, 8-wave GEMM
    (300, 2048, 2048, 8, True, "bf16", "f32", "bf16"),
    (37, 256, 272, 4, True, "f32", "f32", "f32"),
    (16, 8192, 4096, 4, True, "f32", "f32", "bf16"),
    (1, 8192, 1024, 4, True, "f32", "bf16", "bf16"),
    (129, 4096, 512, 4, False, "bf16", "bf16", "bf16"),
    (70, 32768, 96, 8, True, "bf16", "f32", "f32"),
    (0, 2048, 512, 8, True, "bf16", "f32", "bf16"),
    (64, 2048, 8192, 8, True, "f32", "f32", "bf16"),
    (5, 1024, 512, 8, True, "bf16", "bf16", "f32"),
]


@pytest.mark.parametrize("M,K,N,bits,had,xdt,wdt,ydt", LATENT_CASES)
def test_forward_latent_matches_two_calls(M, K, N, bits, had, xdt, wdt, ydt):
    import torch
    _announce("forward_latent M=%d K=%d N=%d a%d had=%d x %s W %s y %s" % (M, K, N, bits, had, xdt, wdt, ydt))
    rng = np.random.default_rng(M + K + N + bits)
    X, _ = workloads.x_outlier_gaussian(rng, max(M, 1), K, 4, 30.0)
    X = X[:M]
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    Wd = to_dev(workloads.f32_to_bf16_bits(W) if wdt == "bf16" else W)
    cfg = hbl.Config(act_bits=bits, hadamard=had)
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    Y, Wp, alpha = hbl.hbl_forward_latent(Xd, Wd, cfg, eps=1e-5, y_dtype=yt)
    Wp2, alpha2 = hbl.hbl_quantize_weights(Wd, eps=1e-5)
    Y2 = hbl.hbl_forward(Xd, Wp2, alpha2, N, cfg, y_dtype=yt)
    _sync()
    assert np.array_equal(to_host(alpha), to_host(alpha2))
    assert np.array_equal(to_host(Wp), to_host(Wp2))
    assert Y.shape == (M, N) and np.array_equal(to_host(Y), to_host(Y2))


def test_forward_deterministic_and_empty():
    import torch
    layer = workloads.WO_1P3B
    X, W, _ = workloads.make_inputs(layer, 3, M=300)
    Xd = to_dev(X)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    cfg = hbl.Config(act_bits=8)
    y1 = to_host(hbl.hbl_forward(Xd, Wp, alpha, layer.N, cfg))
    y2 = to_host(hbl.hbl_forward(Xd, Wp, alpha, layer.N, cfg))
    assert np.array_equal(y1, y2)
    Y0 = hbl.hbl_forward(Xd[:0], Wp, alpha, layer.N, cfg)
    _sync()
    assert Y0.shape == (0, layer.N)


# ====================================================== attention states ==
# Per-(token, head) absmax quantisation to unsigned codes: codes and scales
# bit for bit against the oracle (both sides decide in fp32 with the same
# correctly rounded division and one fp32 product per element), for every
# bit width and head size, both input dtypes, ragged counts of head vectors
# (not a multiple of the block), zero vectors and large magnitudes.
HEAD_CASES = [
    # (M, H, D, bits, x dtype)
    (37, 5, 128, 3, "bf16"), (37, 5, 128, 4, "f32"), (37, 5, 128, 8, "bf16"),
    (3, 7, 32, 3, "f32"), (9, 3, 64, 4, "bf16"), (11, 2, 256, 3, "bf16"), (5, 9, 256, 8, "f32"),
    (1, 1, 32, 3, "bf16"), (2048, 32, 128, 3, "bf16"),
]


@pytest.mark.parametrize("M,H,D,bits,xdt", HEAD_CASES)
def test_quantize_heads_parity(M, H, D, bits, xdt):
    _announce("heads M=%d H=%d D=%d b%d %s" % (M, H, D, bits, xdt))
    rng = np.random.default_rng(M * 7 + H * 3 + D + bits)
    X = (rng.standard_normal((M, H, D)) * rng.choice([0.01, 1.0, 300.0], size=(M, H, 1))).astype(np.float32)
    X[0, 0] = 0.0                                    # a zero head vector
    if M > 1:
        X[1, 0, 5] = 1e30 if xdt == "f32" else 3e38  # one huge element (bf16 keeps its exponent)
    Xh = workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X
    codes, scales = hbl.hbl_quantize_heads(to_dev(Xh), H, bits, eps=1e-5)
    _sync()
    c_ref, d_ref = oracle.quantize_heads(Xh, bits, eps=1e-5)
    assert np.array_equal(to_host(scales), d_ref)
    assert np.array_equal(to_host(codes), c_ref)


def test_quantize_heads_eps_zero_and_ties():
    """eps = 0 puts the extreme element exactly on +-Qp and exact halves on ties
    (round half to even), like the oracle's hand-derived cases."""
    _announce("heads eps=0 ties")
    x = np.array([3.0, 0.5, 1.5, 2.5, -0.5, -2.5, 0.0, 1.0] * 4, np.float32).reshape(1, 1, 32)
    for bits in (3, 4, 8):
        codes, scales = hbl.hbl_quantize_heads(to_dev(x), 1, bits, eps=0.0)
        _sync()
        c_ref, d_ref = oracle.quantize_heads(x, bits, eps=0.0)
        assert np.array_equal(to_host(codes), c_ref) and np.array_equal(to_host(scales), d_ref)


# ============================================================== backward ==
# The straight-through backward against O12: dX within 2e-5 of each row's
# largest |dX| (fp32 transform and sums against fp64), dW within 2e-5 of each
# row's largest |dW| against O12's weight part on the GPU's own codes and
# factors (so a code on a rounding boundary cannot differ); dY in fp32 (split
# into two bf16 parts) and bf16, both norms and none, with and without the
# Hadamard and the gain, INT8 and INT4 codes, ragged M and N (not multiples of
# the 128 x 128 tile), and dX alone.
BWD_CASES = [
    # (M, K, N, bits, hadamard, norm, gain, dY dtype, X dtype)
    (37, 1024, 272, 8, True, hbl.HBL_NORM_RMS, False, "f32", "f32"),
    (130, 2048, 400, 4, True, hbl.HBL_NORM_LN, True, "bf16", "bf16"),
    (64, 512, 64, 8, False, hbl.HBL_NORM_NONE, True, "f32", "bf16"),
    (200, 4096, 128, 4, True, hbl.HBL_NORM_RMS, True, "f32", "f32"),
    (9, 16384, 48, 8, True, hbl.HBL_NORM_RMS, False, "bf16", "f32"),
    (3, 32768, 32, 4, False, hbl.HBL_NORM_LN, False, "f32", "bf16"),
]


def _rowwise_close(got, ref, rel):
    scale = np.maximum(np.max(np.abs(ref), axis=1, keepdims=True), 1e-30)
    return np.all(np.abs(got - ref) <= rel * scale)


@pytest.mark.parametrize("M,K,N,bits,had,norm,use_gain,dydt,xdt", BWD_CASES)
def test_backward_parity(M, K, N, bits, had, norm, use_gain, dydt, xdt):
    _announce("backward M=%d K=%d N=%d a%d had=%d norm=%d gain=%d dY %s X %s" % (M, K, N, bits, had, norm,
                                                                                use_gain, dydt, xdt))
    rng = np.random.default_rng(M + K + N * 3 + bits)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    if norm == hbl.HBL_NORM_LN:
        X = (X + np.float32(2.0)).astype(np.float32)
    W = workloads.w_latent(rng, N, K)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    gain = (rng.standard_normal(K).astype(np.float32) * 0.5 + 1.0) if use_gain else None
    Xh = workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X
    dYh = workloads.f32_to_bf16_bits(dY) if dydt == "bf16" else dY
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=norm)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    gd = None if gain is None else to_dev(gain)
    dX, dW = hbl.hbl_backward(to_dev(dYh), to_dev(Xh), Wp, alpha, cfg, gain=gd)
    codes, _, _, _ = hbl.hbl_quantize_activations(to_dev(Xh), cfg, gain=gd)
    _sync()
    a = to_host(alpha)[0]
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    dX_ref, _ = oracle.backward(dYh, Xh, Wq, a, bits=bits, hadamard=had, gain=gain, norm=norm, want_dW=False)
    assert _rowwise_close(to_host(dX).astype(np.float64), dX_ref, 2e-5)
    q, d = _backward_codes(Xh, to_host(codes), K, bits, had, gain, norm)
    dW_ref = oracle.weight_grad(dYh, q, d)
    check_dw(to_host(dW), dYh, q, d, dW_ref, "dW")


def _backward_codes(Xh, codes_gpu, K, bits, had, gain, norm):
    """The oracle's activation codes and factors for the weight gradient.  A
    code may sit on a rounding boundary that the oracle's fp64 and the GPU's
    fp32 decide differently (by 1, checked); there the weight gradient uses
    the GPU's code, as the forward parity does."""
    ref = oracle.quantize_activations(Xh, bits=bits, hadamard=had, gain=gain, norm=norm)
    q_gpu = unpack_codes(codes_gpu, K, bits)
    check_codes_end_to_end(q_gpu, ref["z"], ref["s"], ref["q"], "backward codes")
    return np.where(q_gpu != ref["q"], q_gpu, ref["q"]), ref["d"]


@pytest.mark.parametrize("M,K,N,bits", [(4096, 2048, 2048, 8), (4100, 4096, 4000, 4)])
def test_backward_large_sampled(M, K, N, bits):
    """Full-size layer (4096 tokens, 2048 x 2048, INT8) and a ragged shape whose
    products both take the 256 x 256 GEMM blocks: 40 sampled rows of dX, 48
    sampled columns of dW, against the oracle."""
    _announce("backward large M=%d K=%d N=%d a%d" % (M, K, N, bits))
    rng = np.random.default_rng(M + K + N)
    X = workloads.f32_to_bf16_bits(workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)[0])
    W = workloads.w_latent(rng, N, K)
    dY = workloads.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    cfg = hbl.Config(act_bits=bits)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    dX, dW = hbl.hbl_backward(to_dev(dY), to_dev(X), Wp, alpha, cfg)
    codes, _, _, _ = hbl.hbl_quantize_activations(to_dev(X), cfg)
    _sync()
    rows = workloads.sample_rows(M, 40)
    cols = np.unique(np.concatenate([np.arange(8), K - 8 + np.arange(8), rng.choice(K, 32, replace=False)]))
    a = to_host(alpha)[0]
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    dX_ref, _ = oracle.backward(dY[rows], X[rows], Wq, a, bits=bits, want_dW=False)
    assert _rowwise_close(to_host(dX)[rows].astype(np.float64), dX_ref, 2e-5)
    q, d = _backward_codes(X, to_host(codes), K, bits, True, None, hbl.HBL_NORM_RMS)
    qc = np.ascontiguousarray(q[:, cols])
    dW_ref = oracle.weight_grad(dY, qc, d)
    check_dw(to_host(dW)[:, cols], dY, qc, d, dW_ref, "dW")


def test_backward_wdown_7b_sampled():
    """The 7B Wdown backward shape the benchmark times (8192 x 16384 -> 4096,
    INT4, bf16 dY): 24 sampled rows of dX against the oracle, 32 sampled
    columns of dW against the oracle's weight gradient on the GPU's own codes
    and factors (identical quantiser inputs; those codes are themselves
    checked against the oracle on the sampled rows), with the M-dependent
    bound of parity.dw_tolerance (8192 tokens: about 5 * 2^-16)."""
    layer = workloads.WDOWN_7B
    M, K, N, bits = layer.M, layer.K, layer.N, layer.act_bits
    _announce("backward wdown_7b M=%d K=%d N=%d a%d" % (M, K, N, bits))
    X, W, _ = workloads.make_inputs(layer, 0)
    rng = np.random.default_rng(11)
    dY = workloads.f32_to_bf16_bits(rng.standard_normal((M, N)).astype(np.float32))
    cfg = hbl.Config(act_bits=bits, hadamard=layer.hadamard)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    Xd = to_dev(X)
    dX, dW = hbl.hbl_backward(to_dev(dY), Xd, Wp, alpha, cfg)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    _sync()
    rows = workloads.sample_rows(M, 24)
    cols = np.unique(np.concatenate([np.arange(4), K - 4 + np.arange(4), rng.choice(K, 24, replace=False)]))
    a = to_host(alpha)[0]
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    dX_rows = to_host(dX)[rows].astype(np.float64)
    dW_cols = np.ascontiguousarray(to_host(dW)[:, cols])
    q_gpu = unpack_codes(to_host(codes), K, bits)
    d_gpu = to_host(xs)
    del dX, dW, Xd
    dX_ref, _ = oracle.backward(dY[rows], X[rows], Wq, a, bits=bits, hadamard=layer.hadamard, want_dW=False)
    assert _rowwise_close(dX_rows, dX_ref, 2e-5)
    ref = oracle.quantize_activations(X[rows], bits=bits, hadamard=layer.hadamard)
    check_codes_end_to_end(q_gpu[rows], ref["z"], ref["s"], ref["q"], "backward codes")
    qc = np.ascontiguousarray(q_gpu[:, cols])
    check_dw(dW_cols, dY, qc, d_gpu, oracle.weight_grad(dY, qc, d_gpu), "dW 7B")


def test_backward_dx_only_and_empty():
    import torch
    _announce("backward dX only, M = 0")
    rng = np.random.default_rng(3)
    M, K, N = 70, 2048, 96
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    W = workloads.w_latent(rng, N, K)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    cfg = hbl.Config(act_bits=8)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    dX, dW = hbl.hbl_backward(to_dev(dY), to_dev(X), Wp, alpha, cfg, want_dW=False)
    dX2, _ = hbl.hbl_backward(to_dev(dY), to_dev(X), Wp, alpha, cfg)
    e = hbl.hbl_backward(to_dev(dY[:0]), to_dev(X[:0]), Wp, alpha, cfg)
    _sync()
    assert dW is None and np.array_equal(to_host(dX), to_host(dX2))
    assert e[0].shape == (0, K)


def test_binding_rejects_small_buffers():
    """Outputs and workspaces smaller than the call needs are refused before
    anything is queued."""
    import torch
    rng = np.random.default_rng(2)
    M, K, N = 8, 1024, 64
    X = to_dev(rng.standard_normal((M, K)).astype(np.float32))
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(workloads.w_latent(rng, N, K)))
    cfg = hbl.Config(act_bits=8)
    small_y = torch.empty((M, N - 1), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ValueError):
        hbl.hbl_forward(X, Wp, alpha, N, cfg, Y=small_y)
    codes, xs, _, _ = hbl.hbl_quantize_activations(X, cfg)
    with pytest.raises(ValueError):
        hbl.hbl_gemm(codes, xs, 8, K, Wp[: N // 2], alpha, N)
    with pytest.raises(ValueError):
        hbl.hbl_backward(to_dev(rng.standard_normal((M, N)).astype(np.float32)), X, Wp, alpha, cfg,
                         dX=torch.empty((M, K - 1), dtype=torch.float32, device="cuda:0"))
    with pytest.raises(hbl.HblError):      # the workspace size is the C ABI's own check
        hbl.hbl_forward(X, Wp, alpha, N, cfg, ws=torch.empty(16, dtype=torch.uint8, device="cuda:0"))
    _sync()
