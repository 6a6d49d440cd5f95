"""Edge cases of the method driven through the HIP path (C ABI) and compared
with the oracle: the closed-form Hadamard column, exact rounding ties, and
rows so small that the quantiser's multiplier overflows fp32 (quant_eps = 0).

The closed form ("新智元: 微软 BitNet v2" repost, section "H-BitLinear模块":
the transform has +-1 entries and orthogonal rows): x = c * h_j, h_j the
column j of the unnormalised Sylvester matrix, gives after RMSNorm and the
normalised transform z = sqrt(K) e_j, so the INT8 codes are 127 e_j, the
INT4 codes 7 e_j, and acc[m][n] = code * W_q[n][j] exactly.
"""
import numpy as np
import pytest
import scipy.linalg

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import check_codes_given_inputs, to_dev, to_host, unpack_codes

pytestmark = pytest.mark.gpu


def _announce(msg):
    print("[case] " + msg, flush=True)


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("K", [256, 2048, 16384])
@pytest.mark.parametrize("bits,a4", [(8, 0), (4, 0), (4, 1)])
def test_closed_form_hadamard_column(K, bits, a4):
    import torch
    _announce("closed form K=%d a%d a4_mode=%d" % (K, bits, a4))
    N = 256
    js = np.array([0, 1, K // 2 + 3, K - 1])
    H = scipy.linalg.hadamard(K) if K <= 2048 else None
    X = np.empty((len(js), K), np.float32)
    for m, j in enumerate(js):
        col = H[:, j] if H is not None else np.array([1 - 2 * (bin(i & int(j)).count("1") & 1) for i in range(K)])
        X[m] = np.float32(0.75 * (1 + m)) * col.astype(np.float32)
    rng = np.random.default_rng(K + bits)
    W = workloads.w_latent(rng, N, K)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W), eps=1e-5)
    cfg = hbl.Config(act_bits=bits, hadamard=True, a4_mode=a4, norm_eps=0.0, quant_eps=0.0)
    for ydt in (torch.float32, torch.bfloat16):
        Y = hbl.hbl_forward(to_dev(X), Wp, alpha, N, cfg, y_dtype=ydt)
        codes, xs, _, _ = hbl.hbl_quantize_activations(to_dev(X), cfg)
        _sync()
        q = unpack_codes(to_host(codes), K, bits)
        top = 127 if bits == 8 else 7
        want = np.zeros_like(q)
        want[np.arange(len(js)), js] = top
        assert np.array_equal(q, want)
        d = to_host(xs)
        # d = gamma/127 = sqrt(K)/127 (INT8), beta/sqrt7 = 1/(sqrt(K) sqrt7) (absmean), sqrt(K)/7 (absmax)
        d_closed = {(8, 0): np.sqrt(K) / 127, (4, 0): 1 / (np.sqrt(K) * np.sqrt(7)), (4, 1): np.sqrt(K) / 7}[(bits, a4)]
        assert np.all(np.abs(d.astype(np.float64) - d_closed) <= 1e-6 * d_closed)
        Wq = oracle.unpack_ternary(to_host(Wp), K)
        acc = top * Wq[:, js].T.astype(np.int32)
        y_ref = oracle.rescale(acc, d, to_host(alpha)[0])
        if ydt == torch.bfloat16:
            y_ref = oracle.f32_to_bf16(y_ref)
        assert np.array_equal(to_host(Y), y_ref)


def _tie_rows(K, rng):
    """Rows z whose products z*s with s = 127/gamma or 7/gamma are exact and
    land on .5 ties (gamma = 127, 63.5 or 7, so s = 1, 2 or 1)."""
    z8 = np.zeros((3, K), np.float32)
    ties = np.arange(-60, 60) + 0.5
    z8[0, :ties.size] = ties
    z8[0, K - 1] = 127.0                       # s = 127/127 = 1
    z8[1, :ties.size] = ties / 2               # s = 127/63.5 = 2: z*s = ties
    z8[1, K - 2] = -63.5
    z8[2] = rng.choice(np.arange(-40, 40) + 0.5, K).astype(np.float32)
    z8[2, 5] = 127.0
    z4 = np.zeros((2, K), np.float32)
    t4 = np.array([-6.5, -5.5, -4.5, -3.5, -2.5, -1.5, -0.5, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5], np.float32)
    z4[0, :t4.size] = t4
    z4[0, K - 1] = 7.0                         # absmax/7: s = 7/7 = 1
    z4[1] = rng.choice(t4, K)
    z4[1, 3] = -7.0
    return z8, z4


@pytest.mark.parametrize("K", [256, 1024, 4096, 16384])
@pytest.mark.parametrize("had", [False, True])
def test_rounding_ties(K, had):
    """Pre-round values exactly on .5: the codes must round half to even, as
    the oracle does.  With the transform on, the input is x = H z (exact for
    these dyadic values when sqrt(K) is a power of two), so the GPU's z is the
    tie row again."""
    _announce("ties K=%d hadamard=%d" % (K, had))
    rng = np.random.default_rng(K)
    z8, z4 = _tie_rows(K, rng)
    for bits, a4, Z in ((8, 0, z8), (4, 1, z4)):
        if had:
            R = np.stack([oracle.hadamard_rows(z[None, :].astype(np.float32))[0] for z in Z]).astype(np.float32)
        else:
            R = Z
        cfg = hbl.Config(act_bits=bits, hadamard=had, norm=hbl.HBL_NORM_NONE, a4_mode=a4, quant_eps=0.0)
        codes, xs, zg, sg = hbl.hbl_quantize_activations(to_dev(np.ascontiguousarray(R)), cfg, z_debug=True,
                                                         s_debug=True)
        _sync()
        zg = to_host(zg)
        assert np.array_equal(zg, Z), "the transform of H z must give z back exactly"
        q = unpack_codes(to_host(codes), K, bits)
        ref = oracle.quantize_activations(R, bits=bits, hadamard=had, norm=oracle.NORM_NONE, quant_eps=0.0,
                                          a4_mode=a4)
        assert np.array_equal(q, ref["q"])
        check_codes_given_inputs(zg, to_host(sg), to_host(xs), q, bits, a4, 0.0, "ties")
        # the ties really are ties, and they went to the even neighbour
        s = to_host(sg).astype(np.float64)
        t = Z.astype(np.float64) * s[:, None]
        on_tie = np.abs(t - np.floor(t) - 0.5) == 0
        assert on_tie.sum() > 50
        assert np.all(q[on_tie] % 2 == 0)


@pytest.mark.parametrize("bits,a4,had,c", [(8, 0, False, 1e-37), (8, 0, True, 1.5e-38), (4, 1, False, 2e-38),
                                           (8, 0, False, 4e-37)])
def test_quant_eps_zero_tiny_rows(bits, a4, had, c):
    """quant_eps = 0 on rows whose statistic is below num / FLT_MAX: the
    multiplier overflows and the row is a zero statistic (codes 0, d = 0, y = 0)
    on both sides; 4e-37 stays finite (127/4e-37 = 3.2e38) and keeps its codes.
    No subnormal value occurs in these rows or in their transforms."""
    import torch
    _announce("tiny rows a%d a4=%d had=%d c=%g" % (bits, a4, had, c))
    K, N = 256, 64
    rng = np.random.default_rng(3)
    X = np.zeros((4, K), np.float32)
    if had:
        H = scipy.linalg.hadamard(K).astype(np.float32)
        for m in range(4):
            X[m] = np.float32(c) * H[:, 7 * m + 1]
    else:
        for m in range(4):
            idx = rng.choice(K, 6, replace=False)
            X[m, idx] = np.float32(c) * rng.choice(np.array([1.0, -1.0, 0.5, -0.75], np.float32), 6)
            X[m, idx[0]] = np.float32(c)
    cfg = hbl.Config(act_bits=bits, hadamard=had, norm=hbl.HBL_NORM_NONE, a4_mode=a4, quant_eps=0.0)
    W = workloads.w_latent(rng, N, K)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W), eps=1e-5)
    Y = hbl.hbl_forward(to_dev(X), Wp, alpha, N, cfg, y_dtype=torch.float32)
    codes, xs, zg, sg = hbl.hbl_quantize_activations(to_dev(X), cfg, z_debug=True, s_debug=True)
    _sync()
    ref = oracle.quantize_activations(X, bits=bits, hadamard=had, norm=oracle.NORM_NONE, quant_eps=0.0, a4_mode=a4)
    q = unpack_codes(to_host(codes), K, bits)
    assert np.array_equal(to_host(zg), ref["z"])
    assert np.array_equal(q, ref["q"])
    assert np.array_equal(to_host(xs), ref["d"])
    assert np.array_equal(to_host(sg), ref["s"])
    zero = c < 3.7e-37 if bits == 8 else True
    assert (not q.any()) == zero
    Wq = oracle.unpack_ternary(to_host(Wp), K)
    assert np.array_equal(to_host(Y), oracle.rescale(oracle.int_gemm(ref["q"], Wq), ref["d"], to_host(alpha)[0]))


def test_quantize_heads_overflowing_multiplier():
    """The head quantiser with eps = 0 on vectors whose Qp / gamma overflows
    fp32: every code at the zero point and d = 0, as the oracle."""
    _announce("heads tiny vectors")
    X = np.zeros((2, 4, 64), np.float32)
    for bits, gamma in ((8, 1e-37), (4, 2e-38)):
        X[:] = 0
        X[:, :, 5] = gamma
        X[:, :, 9] = -gamma / 2
        X[1, 2, 5] = gamma * 40                 # finite multiplier: keeps its codes
        codes, scales = hbl.hbl_quantize_heads(to_dev(X), 4, bits, 0.0)
        _sync()
        c_ref, d_ref = oracle.quantize_heads(X, bits, eps=0.0)
        assert np.array_equal(to_host(codes), c_ref)
        assert np.array_equal(to_host(scales), d_ref)
        assert float(d_ref[0, 0]) == 0.0 and float(d_ref[1, 2]) > 0.0
