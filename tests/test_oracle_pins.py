"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle step against something other than the oracle:
values the pages print (tests/golden), hand-derived cases, closed forms,
library routines (scipy's Sylvester Hadamard, torch's norms, numpy's integer
matmul), invariants, and brute force on tiny inputs.  Together they are chosen
so that a dropped term, a wrong sign or index, a transposed operand, a wrong
rounding mode or a misplaced epsilon in the oracle fails at least one test.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
import workloads


# ------------------------------------------------------------------ Hadamard
@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024])
def test_hadamard_equals_scipy_sylvester(n):
    """O6 against scipy.linalg.hadamard (Sylvester construction, natural order)."""
    rng = np.random.default_rng(n)
    R = rng.standard_normal((3, n))
    H = scipy.linalg.hadamard(n).astype(np.float64) / math.sqrt(n)
    Z = oracle.hadamard_rows(R)
    ref = R @ H.T
    assert np.max(np.abs(Z - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_hadamard_small_explicit(golden):
    g = golden("hadamard_sylvester.txt")
    for key, n in (("H2", 2), ("H4", 4)):
        H = np.array(g[key], np.float64)
        Hor = oracle.hadamard_rows(np.eye(n)).T      # columns = H e_j
        assert np.allclose(Hor * math.sqrt(n), H, atol=1e-14)
    assert oracle.hadamard_rows(np.array([[5.0]]))[0, 0] == 5.0


@pytest.mark.parametrize("n", [8, 64, 256])
def test_hadamard_orthonormal_symmetric(n):
    H = oracle.hadamard_rows(np.eye(n))              # row i = H e_i = column i (H symmetric)
    assert np.allclose(H, H.T, atol=1e-14)
    assert np.allclose(H @ H.T, np.eye(n), atol=1e-12)
    assert np.all(np.isclose(np.abs(H) * math.sqrt(n), 1.0, atol=1e-13))


def test_hadamard_recursive_block_structure():
    """H_2n r = [H_n(a+b), H_n(a-b)] / sqrt(2) for r = [a, b] (natural order)."""
    rng = np.random.default_rng(7)
    for n in (16, 128, 512):
        r = rng.standard_normal(2 * n)
        a, b = r[:n], r[n:]
        z = oracle.hadamard_rows(r[None])[0]
        top = oracle.hadamard_rows((a + b)[None])[0] / math.sqrt(2)
        bot = oracle.hadamard_rows((a - b)[None])[0] / math.sqrt(2)
        assert np.allclose(z, np.concatenate([top, bot]), atol=1e-12)


def test_hadamard_involution_norm_ones():
    rng = np.random.default_rng(3)
    n = 2048
    r = rng.standard_normal((2, n))
    z = oracle.hadamard_rows(r)
    assert np.allclose(oracle.hadamard_rows(z), r, atol=1e-11)           # H H = I
    assert np.allclose(np.linalg.norm(z, axis=1), np.linalg.norm(r, axis=1), rtol=1e-13)
    ones = oracle.hadamard_rows(np.ones((1, n)))[0]                       # H 1 = sqrt(n) e_0
    e0 = np.zeros(n)
    e0[0] = math.sqrt(n)
    assert np.allclose(ones, e0, atol=1e-10)


# ---------------------------------------------------------------------- norm
def test_rmsnorm_matches_torch():
    rng = np.random.default_rng(11)
    X = (rng.standard_normal((5, 96)) * 3).astype(np.float32)
    g = (rng.standard_normal(96) + 1).astype(np.float32)
    for eps in (0.0, 1e-5, 0.25):
        for gain in (None, g):
            r = oracle.norm_rows(X, gain=gain, norm=oracle.NORM_RMS, eps=eps)
            w = None if gain is None else torch.from_numpy(gain.astype(np.float64))
            ref = torch.nn.functional.rms_norm(torch.from_numpy(X.astype(np.float64)), (96,), weight=w, eps=eps)
            assert np.allclose(r, ref.numpy(), rtol=1e-13, atol=1e-13)


def test_layernorm_matches_torch():
    rng = np.random.default_rng(12)
    X = (rng.standard_normal((5, 64)) * 2 + 1.5).astype(np.float32)
    g = (rng.standard_normal(64) + 1).astype(np.float32)
    for eps in (0.0, 1e-5):
        for gain in (None, g):
            r = oracle.norm_rows(X, gain=gain, norm=oracle.NORM_LN, eps=eps)
            w = None if gain is None else torch.from_numpy(gain.astype(np.float64))
            ref = torch.nn.functional.layer_norm(torch.from_numpy(X.astype(np.float64)), (64,), weight=w,
                                                 bias=None, eps=eps)
            assert np.allclose(r, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_norm_hand_and_none():
    r = oracle.norm_rows(np.array([[3.0, 4.0]], np.float32), norm=oracle.NORM_RMS, eps=0.0)[0]
    rms = math.sqrt((9 + 16) / 2)
    assert np.allclose(r, [3 / rms, 4 / rms], rtol=1e-15)
    x = np.array([[1.0, -2.0, 3.0, 0.5]], np.float32)
    g = np.array([2.0, 0.5, -1.0, 4.0], np.float32)
    assert np.array_equal(oracle.norm_rows(x, gain=g, norm=oracle.NORM_NONE)[0], [2.0, -1.0, -3.0, 2.0])


# ------------------------------------------------------------------ weights
def test_ternary_page_example(golden):
    """The bitmask-storage example of the CSDN blog, section 掩码存储."""
    g = golden("ternary_page_example.txt")
    W = np.array(g["latent"], np.float32)
    alpha = oracle.weight_alpha(W)
    assert alpha == np.float32(g["alpha"])
    q = oracle.ternarize(W, alpha, 0.0)
    assert q.tolist() == g["ternary"]
    bitmask = (q != 0).astype(int).tolist()
    signs = [1 if v > 0 else 0 for v in q if v != 0]
    assert bitmask == g["bitmask"] and signs == g["signs"]
    assert len(bitmask) + len(signs) == g["bits"]


def test_ternary_hand_cases(golden):
    g = golden("ternary_hand.txt")
    for key in ("tie", "mean", "eps"):
        W = np.array(g[key + "_latent"], np.float32)
        alpha = oracle.weight_alpha(W)
        assert oracle.ternarize(W, alpha, g[key + "_eps"]).tolist() == g[key + "_ternary"], key
    W = np.array(g["eps_latent"], np.float32)
    assert oracle.ternarize(W, oracle.weight_alpha(W), 0.0).tolist() == g["eps0_ternary"]
    assert oracle.weight_alpha(np.array(g["alpha_tensor"], np.float32)) == np.float32(g["alpha_value"])


def test_ternary_threshold_rule():
    """q = 0 exactly when |W| <= (alpha+eps)/2 (inclusive zero band), sign kept otherwise."""
    rng = np.random.default_rng(5)
    W = (rng.standard_normal(20000) * 0.02).astype(np.float32)
    alpha = oracle.weight_alpha(W)
    q = oracle.ternarize(W, alpha, 0.0)
    t = np.abs(W.astype(np.float64)) / float(alpha)
    clear = np.abs(t - 0.5) > 1e-6
    assert np.array_equal((q == 0)[clear], (t <= 0.5)[clear])
    nz = q != 0
    assert np.array_equal(np.sign(q[nz]), np.sign(W[nz]).astype(np.int8))
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    assert 0.2 < np.mean(q == 0) < 0.45       # Gaussian: P(|w| <= 0.5*mean|w|) ~ 0.31


def test_ternary_scale_invariance():
    rng = np.random.default_rng(6)
    W = rng.standard_normal((4, 64)).astype(np.float32)
    q0 = oracle.quantize_weights(W, eps=0.0)[0]
    for e in (-3, 5):
        Ws = (W * np.float32(2.0 ** e)).astype(np.float32)
        assert np.array_equal(oracle.quantize_weights(Ws, eps=0.0)[0], q0)


def test_pack_ternary_golden(golden):
    g = golden("pack_ternary_k16.txt")
    q = np.array([g["ternary"]], np.int8)
    p = oracle.pack_ternary(q)
    assert p[0].tolist() == g["bytes"]
    assert np.array_equal(oracle.unpack_ternary(p, 16), q)


def test_pack_ternary_roundtrip_and_positions():
    rng = np.random.default_rng(8)
    q = rng.integers(-1, 2, size=(37, 128)).astype(np.int8)
    p = oracle.pack_ternary(q)
    assert p.shape == (37, 32)
    assert np.array_equal(oracle.unpack_ternary(p, 128), q)
    # a single +1 at k lands in byte 4*(k//16) + k%4 at bit pair (k%16)//4
    for k in range(128):
        one = np.zeros((1, 128), np.int8)
        one[0, k] = 1
        pk = oracle.pack_ternary(one)[0]
        expect = np.zeros(32, np.uint8)
        expect[4 * (k // 16) + k % 4] = 1 << (2 * ((k % 16) // 4))
        assert np.array_equal(pk, expect), k
    # the code 10 never appears
    bits = np.unpackbits(p.reshape(-1, 1), axis=1, bitorder="little").reshape(-1, 4, 2)
    assert not np.any((bits[:, :, 0] == 0) & (bits[:, :, 1] == 1))


def test_quantize_weights_composition():
    rng = np.random.default_rng(9)
    W = workloads.w_latent(rng, 48, 64)
    Wq, Wp, alpha = oracle.quantize_weights(W, eps=1e-5)
    assert alpha == oracle.weight_alpha(W)
    assert abs(float(alpha) - float(np.mean(np.abs(W.astype(np.float64))))) <= 1e-7 * float(alpha)
    assert np.array_equal(Wq, oracle.ternarize(W, alpha, 1e-5))
    assert np.array_equal(oracle.unpack_ternary(Wp, 64), Wq)
    with pytest.raises(ValueError):
        oracle.quantize_weights(W[:, :40])      # K % 16 != 0


# -------------------------------------------------------------- activations
def test_int8_hand_cases(golden):
    g = golden("act_quant_hand.txt")
    for key in ("i8_a", "i8_b", "i8_c", "i8_d"):
        z = np.array(g[key + "_z"], np.float32)
        s, d = oracle.act_scale(z, 8, eps=g[key + "_eps"])
        assert oracle.act_codes(z, 8, s).tolist() == g[key + "_codes"], key
        gamma = np.max(np.abs(z))
        assert d == np.float32(gamma / np.float32(127.0))
    s, _ = oracle.act_scale(np.array(g["i8_a_z"], np.float32), 8, eps=0.0)
    assert s == np.float32(g["i8_a_s"])


def test_int4_hand_cases(golden):
    g = golden("act_quant_hand.txt")
    sqrt7 = np.float32(math.sqrt(7.0))
    for key in ("i4_a", "i4_b", "i4_c", "i4_d"):
        z = np.array(g[key + "_z"], np.float32)
        s, d = oracle.act_scale(z, 4, a4_mode=oracle.A4_ABSMEAN, eps=0.0)
        assert oracle.act_codes(z, 4, s).tolist() == g[key + "_codes"], key
        beta = np.float32(np.mean(np.abs(z.astype(np.float64))))
        assert s == np.float32(sqrt7 / beta) and d == np.float32(beta / sqrt7)
    z = np.array(g["i4m_z"], np.float32)
    s, d = oracle.act_scale(z, 4, a4_mode=oracle.A4_ABSMAX, eps=0.0)
    assert s == np.float32(1.75) and d == np.float32(np.float32(4.0) / np.float32(7.0))
    assert oracle.act_codes(z, 4, s).tolist() == g["i4m_codes"]


def test_int4_pack_golden(golden):
    g = golden("act_quant_hand.txt")
    q = np.array([g["pack4_codes"]], np.int8)
    p = oracle.pack_int4(q)
    assert p[0].tolist() == g["pack4_bytes"]
    assert np.array_equal(oracle.unpack_int4(p, 4), q)
    rng = np.random.default_rng(2)
    q = rng.integers(-8, 8, size=(9, 64)).astype(np.int8)
    assert np.array_equal(oracle.unpack_int4(oracle.pack_int4(q), 64), q)


def test_act_quant_invariants():
    rng = np.random.default_rng(13)
    for _ in range(20):
        z = (rng.standard_normal(256) * rng.uniform(0.01, 100)).astype(np.float32)
        s, _ = oracle.act_scale(z, 8, eps=0.0)
        q = oracle.act_codes(z, 8, s)
        am = np.argmax(np.abs(z))
        assert abs(int(q[am])) == 127 and np.sign(q[am]) == np.sign(z[am])
        assert q.min() >= -127 and q.max() <= 127
        assert np.array_equal(oracle.act_codes(-z, 8, s), -q)                    # odd symmetry
        z2 = (z * np.float32(8.0)).astype(np.float32)
        assert np.array_equal(oracle.act_codes(z2, 8, oracle.act_scale(z2, 8, eps=0.0)[0]), q)
        s4, _ = oracle.act_scale(z, 4, eps=0.0)
        q4 = oracle.act_codes(z, 4, s4)
        assert q4.min() >= -8 and q4.max() <= 7
        z4 = (z * np.float32(0.25)).astype(np.float32)
        assert np.array_equal(oracle.act_codes(z4, 4, oracle.act_scale(z4, 4, eps=0.0)[0]), q4)
    s, d = oracle.act_scale(np.zeros(64, np.float32), 8, eps=1e-5)          # all-zero row
    assert s == 0 and d == 0
    assert not oracle.act_codes(np.zeros(64, np.float32), 8, s).any()


# --------------------------------------------------------------- int GEMM
def test_int_gemm_matches_numpy():
    rng = np.random.default_rng(21)
    q = rng.integers(-128, 128, size=(7, 96)).astype(np.int8)
    w = rng.integers(-1, 2, size=(11, 96)).astype(np.int8)
    acc = oracle.int_gemm(q, w)
    ref = q.astype(np.int64) @ w.astype(np.int64).T
    assert acc.shape == (7, 11) and np.array_equal(acc, ref)


def test_int_gemm_brute_force_tiny():
    """Every ternary row of length 4 against every INT4 code in each position."""
    import itertools
    rows = np.array(list(itertools.product([-1, 0, 1], repeat=4)), np.int8)      # 81 x 4
    codes = np.array(list(itertools.product(range(-8, 8), repeat=2)), np.int8)   # 256 x 2
    q = np.concatenate([codes, codes[::-1]], axis=1)                             # 256 x 4
    acc = oracle.int_gemm(q, rows)
    for m in range(0, 256, 17):
        for n in range(81):
            assert acc[m, n] == sum(int(q[m, k]) * int(rows[n, k]) for k in range(4))


def test_int_gemm_identity_and_ones():
    rng = np.random.default_rng(22)
    q = rng.integers(-128, 128, size=(5, 16)).astype(np.int8)
    assert np.array_equal(oracle.int_gemm(q, np.eye(16, dtype=np.int8)), q.astype(np.int32))
    assert np.array_equal(oracle.int_gemm(q, np.ones((3, 16), np.int8))[:, 0], q.astype(np.int64).sum(1))


def test_rescale_hand():
    y = oracle.rescale(np.array([[3, -5, 0]], np.int32), np.array([0.5], np.float32), 0.25)
    assert y.tolist() == [[0.375, -0.625, 0.0]]


def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    rows = []
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _fp32_rne(x):
    """Round a nonzero rational to the nearest fp32 (ties to even) with exact
    integer arithmetic; normal range only.  Returns the bit pattern."""
    from fractions import Fraction
    neg = x < 0
    x = abs(Fraction(x))
    e = 0
    while x >= Fraction(2 ** 24) * Fraction(2) ** e:
        e += 1
    while x < Fraction(2 ** 23) * Fraction(2) ** e:
        e -= 1
    m = x / Fraction(2) ** e
    fl = m.numerator // m.denominator
    r = m - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2):
        fl += 1
    if fl == 2 ** 24:
        fl, e = 2 ** 23, e + 1
    return (int(neg) << 31) | ((e + 23 + 127) << 23) | (fl - 2 ** 23)


def test_rescale_rounding_order_golden():
    """y = fp32(fp32(acc*d)*alpha), the factor d first: hand-derived cases
    (tests/golden/rescale_order.txt) where acc*fp32(d*alpha) and the exact
    triple product round to a neighbouring fp32; the expected bits are derived
    again here from exact fractions."""
    from fractions import Fraction
    for acc, dh, ah, yh, other in _golden_rows("rescale_order.txt"):
        acc = int(acc)
        d = np.array([int(dh, 16)], np.uint32).view(np.float32)
        a = np.array([int(ah, 16)], np.uint32).view(np.float32)[0]
        y = oracle.rescale(np.array([[acc]], np.int32), d, a)
        assert int(y.view(np.uint32)[0, 0]) == int(yh, 16)
        t = _fp32_rne(acc * Fraction(float(d[0])))
        t_val = Fraction(float(np.array([t], np.uint32).view(np.float32)[0]))
        assert _fp32_rne(t_val * Fraction(float(a))) == int(yh, 16)
        assert _fp32_rne(acc * Fraction(float(d[0])) * Fraction(float(a))) == int(other, 16) != int(yh, 16)


def test_rescale_rounding_order_random():
    """The same rounding order on 20000 random (acc, d, alpha), each checked
    against the exact-fraction derivation of fp32(fp32(acc*d)*alpha)."""
    from fractions import Fraction
    rng = np.random.default_rng(31)
    acc = rng.integers(-2 ** 20, 2 ** 20, size=(200, 100)).astype(np.int32)
    acc[acc == 0] = 1
    d = rng.uniform(1e-3, 1.0, 200).astype(np.float32)
    a = np.float32(rng.uniform(1e-3, 0.1))
    y = oracle.rescale(acc, d, a).view(np.uint32)
    fa = Fraction(float(a))
    for m in range(200):
        fd = Fraction(float(d[m]))
        for n in range(0, 100, 7):
            t = _fp32_rne(int(acc[m, n]) * fd)
            tv = Fraction(float(np.array([t], np.uint32).view(np.float32)[0]))
            assert int(y[m, n]) == _fp32_rne(tv * fa)


def test_bf16_rounding_golden():
    """fp32 -> bf16 of the bf16 output variant: hand-derived ties (both ways,
    both signs), values just above and below a tie, subnormals, overflow of
    the largest finite values to infinity (tests/golden/bf16_rne.txt)."""
    rows = _golden_rows("bf16_rne.txt")
    x = np.array([int(r[0], 16) for r in rows], np.uint32).view(np.float32)
    want = [int(r[1], 16) for r in rows]
    assert oracle.f32_to_bf16(x).tolist() == want


def test_bf16_rounding_matches_torch():
    """Against torch's fp32 -> bf16 conversion (a library routine, round to
    nearest even) on 400k values: random bit patterns of every exponent
    (NaN excluded, outside the contract), exact ties, and ties with the top
    half odd and even."""
    rng = np.random.default_rng(32)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]                 # no inf / NaN in the random part
    ties = (rng.integers(0, 2 ** 16, size=100000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    near = np.concatenate([ties - 1, ties + 1])
    allb = np.concatenate([bits, ties, near]).astype(np.uint32)
    x = allb.view(np.float32)
    got = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_act_scale_overflow_is_zero_statistic():
    """eps = 0 and a statistic so small that s = num/stat overflows fp32: the
    row is treated as a zero statistic (s = d = 0, codes 0).  127/1e-37 and
    7/2e-38 exceed the largest fp32 (3.4028e38); 127/4e-37 = 3.175e38 does not,
    so that row keeps its codes (the absmax element maps to 127)."""
    z = np.array([[1e-37, 0.0, -5e-38, 0.0]], np.float32)
    s, d = oracle.act_scale(z, 8, eps=0.0)
    assert float(s) == 0.0 and float(d) == 0.0
    assert oracle.act_codes(z, 8, float(s)).tolist() == [0, 0, 0, 0]
    z2 = np.array([[2e-38, 0.0, -1.5e-38, 0.0]], np.float32)
    s2, d2 = oracle.act_scale(z2, 4, a4_mode=oracle.A4_ABSMAX, eps=0.0)
    assert float(s2) == 0.0 and float(d2) == 0.0
    z3 = np.array([[4e-37, 0.0, -2e-37, 0.0]], np.float32)
    s3, d3 = oracle.act_scale(z3, 8, eps=0.0)
    assert np.isfinite(s3) and float(s3) > 3.0e38
    assert oracle.act_codes(z3, 8, float(s3)).tolist() == [127, 0, -64, 0]
    r = oracle.quantize_activations(np.array([[1e-37, 0, -5e-38, 0] * 64], np.float32), bits=8, hadamard=False,
                                    norm=oracle.NORM_NONE, quant_eps=0.0)
    assert not r["q"].any() and float(r["d"][0]) == 0.0


def test_heads_scale_overflow_is_zero_vector():
    """The head quantiser under the same reading: gamma with qp/gamma above the
    largest fp32 (eps = 0) gives d = 0 and every code at the zero point."""
    # qp / FLT_MAX: 8.8e-39 (3 bits, subnormal), 2.06e-38 (4 bits), 3.73e-37 (8 bits)
    for bits, gamma in ((3, 8e-39), (4, 2e-38), (8, 1e-37)):
        x = np.zeros((1, 2, 32), np.float32)
        x[0, :, 3] = gamma
        x[0, :, 5] = -gamma / 2
        x[0, 1, 3] = gamma * 20          # qp / gamma finite: keeps its codes
        codes, d = oracle.quantize_heads(x, bits, eps=0.0)
        u = oracle.unpack_heads(codes, 32, bits)
        assert float(d[0, 0]) == 0.0 and (u[0, 0] == 1 << (bits - 1)).all()
        assert float(d[0, 1]) > 0.0 and int(u[0, 1, 3]) == (1 << bits) - 1


# --------------------------------------------------------------- end to end
@pytest.mark.parametrize("K", [256, 1024, 4096])
def test_forward_closed_form_hadamard_column(K):
    """x = c * (column j of the unnormalised Sylvester H): RMSNorm gives the +-1
    column, the normalised H maps it to sqrt(K) e_j, so INT8 codes are 127 e_j
    and y[n] = sqrt(K) * alpha * W_q[n, j] (up to the two fp32 roundings)."""
    rng = np.random.default_rng(K)
    N = 24
    W = workloads.w_latent(rng, N, K)
    Wq, _, alpha = oracle.quantize_weights(W, eps=1e-5)
    Hs = scipy.linalg.hadamard(K)
    for j in (0, 1, K // 2 + 3, K - 1):
        x = (Hs[:, j] * 2.5).astype(np.float32)[None, :]
        out = oracle.forward(x, Wq, alpha, bits=8, quant_eps=0.0, norm_eps=0.0)
        e = np.zeros(K, np.int8)
        e[j] = 127
        assert np.array_equal(out["q"][0], e)
        zref = np.zeros(K)
        zref[j] = math.sqrt(K)
        assert np.allclose(out["z"][0], zref, rtol=1e-6, atol=1e-5)
        assert np.array_equal(out["acc"][0], 127 * Wq[:, j].astype(np.int32))
        assert np.allclose(out["y"][0], math.sqrt(K) * float(alpha) * Wq[:, j], rtol=2e-7, atol=0)
        # INT4 absmean on the same row: beta = 1/sqrt(K), the spike clips at 7
        out4 = oracle.forward(x, Wq, alpha, bits=4, quant_eps=0.0, norm_eps=0.0)
        e4 = np.zeros(K, np.int8)
        e4[j] = 7
        assert np.array_equal(out4["q"][0], e4)


def test_forward_plain_bitlinear_and_bf16():
    """hadamard=0 skips O6; bf16 inputs convert exactly (0x3F80 = 1.0, 0xC000 = -2, 0x3F81 = 1+2^-7)."""
    assert oracle.bf16_to_f32(np.array([0x3F80, 0xC000, 0x3F81], np.uint16)).tolist() == [1.0, -2.0, 1.0078125]
    rng = np.random.default_rng(31)
    X = rng.standard_normal((3, 64)).astype(np.float32)
    qa = oracle.quantize_activations(X, bits=8, hadamard=False)
    r = oracle.norm_rows(X).astype(np.float32)
    assert np.array_equal(qa["z"], r)
    Xb = workloads.f32_to_bf16_bits(X)
    qb = oracle.quantize_activations(Xb, bits=8, hadamard=True)
    qf = oracle.quantize_activations(workloads.bf16_bits_to_f32(Xb), bits=8, hadamard=True)
    assert np.array_equal(qb["q"], qf["q"]) and np.array_equal(qb["z"], qf["z"])


def test_forward_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.quantize_activations(np.zeros((2, 96), np.float32), bits=8, hadamard=True)   # not a power of two
    with pytest.raises(ValueError):
        oracle.quantize_activations(np.zeros((2, 64), np.float32), bits=5)


# ------------------------------------------------ low-bit attention states (O11)
def test_heads_hand_cases(golden):
    g = golden("head_quant_hand.txt")
    x = np.array(g["x"], np.float32).reshape(1, 1, 8)
    for bits, key in ((3, "b3"), (4, "b4"), (8, "b8")):
        codes, d = oracle.quantize_heads(x, bits, eps=0.0)
        assert oracle.unpack_heads(codes, 8, bits).ravel().tolist() == g[key + "_codes"]
        if bits != 8:
            assert codes.ravel().tolist() == g[key + "_bytes"]
        assert d[0, 0] == np.float32(1.0) / np.float32((1 << (bits - 1)) - 1)
    codes, d = oracle.quantize_heads(np.zeros((1, 1, 8), np.float32), 3, eps=0.0)
    assert d[0, 0] == 0.0 and oracle.unpack_heads(codes, 8, 3).ravel().tolist() == g["zero_b3_codes"]
    codes, d = oracle.quantize_heads(np.array(g["ties_x"], np.float32).reshape(1, 1, 8), 3, eps=0.0)
    assert oracle.unpack_heads(codes, 8, 3).ravel().tolist() == g["ties_b3_codes"] and d[0, 0] == 1.0


@pytest.mark.parametrize("bits", [3, 4, 8])
def test_heads_properties(bits):
    """Range, the extreme element, reconstruction within half a step, sign
    symmetry u(-x) = 2^b - u(x), and per-head independence."""
    rng = np.random.default_rng(bits)
    X = rng.standard_normal((5, 3, 64)).astype(np.float32)
    X[1, 2] *= 100.0
    zp, qp = 1 << (bits - 1), (1 << (bits - 1)) - 1
    codes, d = oracle.quantize_heads(X, bits, eps=0.0)
    u = oracle.unpack_heads(codes, 64, bits).astype(np.int64)
    assert u.min() >= 1 and u.max() <= 2 * zp - 1
    q = u - zp
    amax = np.argmax(np.abs(X), axis=2)
    ext = np.take_along_axis(q, amax[..., None], axis=2)[..., 0]
    assert np.array_equal(np.abs(ext), np.full(ext.shape, qp))
    err = np.abs(X.astype(np.float64) - q * d[..., None].astype(np.float64))
    assert np.all(err <= 0.5 * d[..., None] * (1 + 1e-6) + 1e-12)
    codes_n, d_n = oracle.quantize_heads(-X, bits, eps=0.0)
    assert np.array_equal(d_n, d)
    assert np.array_equal(oracle.unpack_heads(codes_n, 64, bits).astype(np.int64), 2 * zp - u)
    one, d1 = oracle.quantize_heads(X[1:2, 2:3], bits, eps=0.0)
    assert np.array_equal(one[0, 0], codes[1, 2]) and d1[0, 0] == d[1, 2]


def test_heads_packing_brute_force():
    """3- and 4-bit packing against bit strings assembled by hand in Python."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((2, 2, 16)).astype(np.float32)
    for bits in (3, 4):
        codes, _ = oracle.quantize_heads(X, bits, eps=1e-5)
        u = oracle.unpack_heads(codes, 16, bits)
        for m in range(2):
            for h in range(2):
                bitstr = sum(int(c) << (bits * j) for j, c in enumerate(u[m, h]))
                assert codes[m, h].tolist() == list(bitstr.to_bytes(16 * bits // 8, "little"))


def test_heads_eps_in_denominator():
    """s = Qp/(gamma+eps): with eps the extreme element no longer lands exactly on Qp."""
    x = np.array([[[2.0, 1.0, 0.5, 0.0, 0.0, 0.0, 0.0, -1.5]]], np.float32)
    c0, _ = oracle.quantize_heads(x, 8, eps=0.0)
    c1, _ = oracle.quantize_heads(x, 8, eps=0.5)
    u0 = oracle.unpack_heads(c0, 8, 8).ravel().astype(int) - 128
    u1 = oracle.unpack_heads(c1, 8, 8).ravel().astype(int) - 128
    assert u0.tolist()[:3] == [127, 64, 32]          # 2*63.5 = 127, 63.5 -> 64 (half even), 31.75 -> 32
    assert u1.tolist()[:3] == [102, 51, 25]          # s = 127/2.5 = 50.8: 101.6, 50.8, 25.4


# ------------------------------------------------ straight-through backward (O12)
def _surrogate_y(x, Wq, alpha, gain, norm, eps, hadamard):
    """fp64 forward of the layer with both quantisers removed (what the
    straight-through backward differentiates), written here with numpy and
    scipy independently of the oracle."""
    x = np.asarray(x, np.float64)
    g = 1.0 if gain is None else np.asarray(gain, np.float64)
    if norm == oracle.NORM_RMS:
        r = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps) * g
    elif norm == oracle.NORM_LN:
        c = x - x.mean(axis=1, keepdims=True)
        r = c / np.sqrt((c * c).mean(axis=1, keepdims=True) + eps) * g
    else:
        r = x * g
    K = x.shape[1]
    z = r @ (scipy.linalg.hadamard(K).astype(np.float64) / math.sqrt(K)).T if hadamard else r
    return alpha * (z @ np.asarray(Wq, np.float64).T)


@pytest.mark.parametrize("norm", [oracle.NORM_RMS, oracle.NORM_LN, oracle.NORM_NONE])
@pytest.mark.parametrize("hadamard,use_gain", [(True, False), (True, True), (False, True)])
def test_backward_dx_finite_differences(norm, hadamard, use_gain):
    """O12's dX equals the central finite-difference gradient of
    sum(dY * y) for the quantiser-free forward."""
    rng = np.random.default_rng(norm * 10 + hadamard * 2 + use_gain)
    M, K, N = 3, 16, 5
    X = (rng.standard_normal((M, K)) + (1.5 if norm == oracle.NORM_LN else 0.0)).astype(np.float32)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    gain = (rng.standard_normal(K) * 0.5 + 1.0).astype(np.float32) if use_gain else None
    alpha, eps = np.float32(0.37), float(np.float32(1e-5))
    dX, _ = oracle.backward(dY, X, Wq, alpha, bits=8, hadamard=hadamard, gain=gain, norm=norm, want_dW=False)
    h = 1e-6
    fd = np.empty((M, K))
    for m in range(M):
        for j in range(K):
            xp = X.astype(np.float64); xm = X.astype(np.float64)
            xp[m, j] += h; xm[m, j] -= h
            lp = np.sum(dY.astype(np.float64) * _surrogate_y(xp, Wq, float(alpha), gain, norm, eps, hadamard))
            lm = np.sum(dY.astype(np.float64) * _surrogate_y(xm, Wq, float(alpha), gain, norm, eps, hadamard))
            fd[m, j] = (lp - lm) / (2 * h)
    assert np.allclose(dX, fd, rtol=1e-6, atol=1e-7 * np.max(np.abs(fd)))


def test_backward_dw_finite_differences():
    """O12's dW equals the gradient of sum(dY * (xh W^T)) in W, with xh = d*q
    the dequantised codes of the forward."""
    rng = np.random.default_rng(5)
    M, K, N = 4, 16, 3
    X = rng.standard_normal((M, K)).astype(np.float32)
    Wq = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    for bits in (8, 4):
        _, dW = oracle.backward(dY, X, Wq, 0.5, bits=bits)
        qa = oracle.quantize_activations(X, bits=bits)
        xh = qa["q"].astype(np.float64) * qa["d"].astype(np.float64)[:, None]
        W0 = rng.standard_normal((N, K))
        fd = np.empty((N, K))
        for n in range(N):
            for k in range(K):
                Wp = W0.copy(); Wm = W0.copy()
                Wp[n, k] += 0.5; Wm[n, k] -= 0.5
                fd[n, k] = (np.sum(dY * (xh @ Wp.T)) - np.sum(dY * (xh @ Wm.T))) / 1.0
        assert np.allclose(dW, fd, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------ base-3 storage (O13)
def test_base3_hand_packed(golden):
    g = golden("pack_base3_k16.txt")
    W = np.array([g["ternary"]], np.int8)
    b = oracle.pack_base3(W)
    assert b[0].tolist() == g["bytes"]
    assert oracle.unpack_base3(b, 16).tolist() == W.tolist()


def test_base3_every_digit_group():
    """All 3^5 groups of five weights: each byte equals Python's own parse of
    the digits t + 1 as a base-3 numeral (most significant digit = last
    weight), so the bytes are 0..242, each exactly once."""
    groups = list(itertools.product((-1, 0, 1), repeat=5))
    W = np.array([t for grp in groups for t in grp], np.int8)[None, :]     # K = 1215
    b = oracle.pack_base3(W)[0]
    for j, grp in enumerate(groups):
        assert b[j] == int("".join(str(t + 1) for t in reversed(grp)), 3)
    assert sorted(b[:243].tolist()) == list(range(243))
    assert np.all(b[243:] == 121) and b.size == 16 * math.ceil(1215 / 80)
    assert np.array_equal(oracle.unpack_base3(oracle.pack_base3(W), 1215), W)


@pytest.mark.parametrize("K", [16, 80, 96, 1024, 8192, 4000])
def test_base3_round_trip_and_padding(K):
    rng = np.random.default_rng(K)
    W = rng.integers(-1, 2, size=(5, K)).astype(np.int8)
    b = oracle.pack_base3(W)
    assert b.shape == (5, 16 * ((K + 79) // 80)) and b.max() <= 242
    assert np.array_equal(oracle.unpack_base3(b, K), W)
    # a byte is a function of its own five weights only
    W2 = W.copy()
    W2[:, 7] = -W2[:, 7] if np.any(W2[:, 7]) else 1
    b2 = oracle.pack_base3(W2)
    changed = np.nonzero(np.any(b2 != b, axis=0))[0]
    assert changed.tolist() == [1]
    # the padding weights past K are zero: all-zero rows are all 121
    assert np.all(oracle.pack_base3(np.zeros((2, K), np.int8)) == 121)


def test_base3_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.pack_base3(np.array([[2, 0, 0, 0]], np.int8))
    bad = oracle.pack_base3(np.zeros((1, 16), np.int8))
    bad[0, 0] = 243
    with pytest.raises(ValueError):
        oracle.unpack_base3(bad, 16)
    bad[0, 0] = 121
    bad[0, 3] = 124        # digits 1,2,1,1,1: k = 15 is 0, the padding weight k = 16 is +1
    with pytest.raises(ValueError):
        oracle.unpack_base3(bad, 16)


# ------------------------------------------------------------- FP4 (O14) ----
def _e2m1_value(nib):
    """Value of a 4-bit E2M1 code from the format's definition (sign bit 3,
    exponent bits 2..1 with bias 1, mantissa bit 0; exponent 0 is subnormal)."""
    sign = -1.0 if nib & 8 else 1.0
    e, m = (nib >> 1) & 3, nib & 1
    return sign * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m))


def test_pack_fp4_golden():
    path = __import__("os").path.join(__import__("os").path.dirname(__file__), "golden", "pack_fp4_k8.txt")
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if "=" in line:
                k, v = line.split("=", 1)
                vals[k.strip()] = v.split()
    wq = np.array([[int(t) for t in vals["weights"]]], np.int8)
    assert oracle.pack_fp4(wq).tolist() == [[int(b, 16) for b in vals["bytes"]]]


def test_pack_fp4_decodes_to_the_ternary_values():
    """Every nibble decodes (E2M1 definition) to its weight, at every position,
    and the low nibble holds the even k."""
    rng = np.random.default_rng(41)
    wq = rng.integers(-1, 2, size=(7, 96)).astype(np.int8)
    p = oracle.pack_fp4(wq)
    dec = np.array([[_e2m1_value((p[n, k // 2] >> (4 * (k % 2))) & 15) for k in range(96)] for n in range(7)])
    assert np.array_equal(dec, wq.astype(np.float64))
    one = np.zeros((1, 16), np.int8)
    one[0, 5] = -1
    assert oracle.pack_fp4(one)[0].tolist() == [0, 0, 0xA0, 0, 0, 0, 0, 0]
