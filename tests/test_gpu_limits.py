"""Size limits of the C ABI.  The largest M the GEMM admits (2^23 rows) and
an activation quantisation whose input passes 2^31 bytes.  The largest output
width, N = 2^20 columns, on every GEMM path: the one-token GEMV, the decode GEMM, the prefill GEMM (INT8 and INT4,
ragged M), the FP6 x FP4 GEMM inside hbl_forward, and base-3 packing and its
GEMV.  At this width a
128-row output tile spans 512 MiB (fp32), the edge of the kernels' 32-bit
tile offsets.  Outputs are checked bit for bit against the oracle's integer
product and rescale on sampled columns, the first and last 16 included.
Weights are random valid 2-bit bytes (each field 00, 01 or 11), so no
ternarisation of 2^20 rows is needed on the host."""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import oracle
import workloads
from parity import to_dev, to_host, unpack_codes

pytestmark = pytest.mark.gpu

NMAX = 1 << 20
_VALID = np.array([a | b << 2 | c << 4 | d << 6 for a in (0, 1, 3) for b in (0, 1, 3) for c in (0, 1, 3)
                   for d in (0, 1, 3)], np.uint8)


def _cols(rng):
    return np.unique(np.concatenate([np.arange(16), NMAX - 16 + np.arange(16), rng.choice(NMAX, 96, replace=False)]))


def _sampled(Y, cols):
    import torch
    return to_host(Y.index_select(1, torch.from_numpy(cols).to(Y.device)).contiguous())


@pytest.mark.parametrize("M,K,bits,ydt", [(3, 1024, 4, "bf16"), (40, 256, 8, "f32"), (40, 128, 4, "bf16"),
                                          (200, 128, 4, "f32"), (130, 256, 8, "bf16")])
def test_gemm_max_width(M, K, bits, ydt):
    import torch
    print("[case] gemm N=2^20 M=%d K=%d a%d %s" % (M, K, bits, ydt), flush=True)
    rng = np.random.default_rng(M * 7 + K + bits)
    Wp = _VALID[rng.integers(0, len(_VALID), size=(NMAX, K // 4), dtype=np.uint8)]
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    q = rng.integers(lo, hi + 1, size=(M, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) * np.float32(0.02) + np.float32(1e-3)).astype(np.float32)
    alpha = np.array([0.0211], np.float32)
    Y = hbl.hbl_gemm(to_dev(q if bits == 8 else oracle.pack_int4(q)), to_dev(d), bits, K, to_dev(Wp), to_dev(alpha),
                     NMAX, y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    cols = _cols(rng)
    y_ref = oracle.rescale(oracle.int_gemm(q, oracle.unpack_ternary(np.ascontiguousarray(Wp[cols]), K)), d, alpha[0])
    got = _sampled(Y, cols)
    assert np.array_equal(got, y_ref if ydt == "f32" else oracle.f32_to_bf16(y_ref))


def test_forward_f6f4_max_width():
    """hbl_forward with the larger workspace (FP6 codes, FP4 weights) at
    N = 2^20: the same output bits as the oracle's product and rescale of the
    GPU's own INT4 codes."""
    import torch
    M, K = 300, 512
    print("[case] forward FP6 x FP4 N=2^20 M=%d K=%d" % (M, K), flush=True)
    rng = np.random.default_rng(2)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    Wp = _VALID[rng.integers(0, len(_VALID), size=(NMAX, K // 4), dtype=np.uint8)]
    alpha = np.array([0.0173], np.float32)
    cfg = hbl.Config(act_bits=4)
    Xd = to_dev(X)
    ws = torch.empty(hbl.hbl_forward_workspace_bytes(M, K, NMAX, cfg), dtype=torch.uint8, device="cuda:0")
    Y = hbl.hbl_forward(Xd, to_dev(Wp), to_dev(alpha), NMAX, cfg, y_dtype=torch.bfloat16, ws=ws)
    codes, xs, _, _ = hbl.hbl_quantize_activations(Xd, cfg)
    torch.cuda.synchronize()
    cols = _cols(rng)
    q = unpack_codes(to_host(codes), K, 4)
    y_ref = oracle.rescale(oracle.int_gemm(q, oracle.unpack_ternary(np.ascontiguousarray(Wp[cols]), K)),
                           to_host(xs), alpha[0])
    assert np.array_equal(_sampled(Y, cols), oracle.f32_to_bf16(y_ref))


@pytest.mark.parametrize("M,K,bits", [(1, 160, 8), (4, 1040, 4)])
def test_base3_max_width(M, K, bits):
    """Base-3 storage at N = 2^20: hbl_pack_base3's bytes on sampled rows
    against the oracle's packing, and hbl_gemm_base3 bit for bit against the
    oracle's product and rescale on sampled columns."""
    import torch
    print("[case] base3 N=2^20 M=%d K=%d a%d" % (M, K, bits), flush=True)
    rng = np.random.default_rng(M + K)
    Wp = _VALID[rng.integers(0, len(_VALID), size=(NMAX, K // 4), dtype=np.uint8)]
    W3 = hbl.hbl_pack_base3(to_dev(Wp), K)
    lo, hi = (-128, 127) if bits == 8 else (-8, 7)
    q = rng.integers(lo, hi + 1, size=(M, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) * np.float32(0.02) + np.float32(1e-3)).astype(np.float32)
    alpha = np.array([0.0211], np.float32)
    Y = hbl.hbl_gemm_base3(to_dev(q if bits == 8 else oracle.pack_int4(q)), to_dev(d), bits, K, W3, to_dev(alpha),
                           NMAX, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cols = _cols(rng)
    Wq = oracle.unpack_ternary(np.ascontiguousarray(Wp[cols]), K)
    assert np.array_equal(to_host(W3.index_select(0, torch.from_numpy(cols).to(W3.device))), oracle.pack_base3(Wq))
    y_ref = oracle.rescale(oracle.int_gemm(q, Wq), d, alpha[0])
    assert np.array_equal(_sampled(Y, cols), oracle.f32_to_bf16(y_ref))


def test_gemm_max_rows():
    """hbl_gemm at M = 2^23 rows (the largest it admits; 1 GiB of INT8 codes),
    bit for bit on sampled rows, the first and last 8 included.  The codes are
    drawn on the GPU by a seeded generator; only the sampled rows come back."""
    import torch
    M, K, N = 1 << 23, 128, 16
    print("[case] gemm M=2^23 K=%d N=%d a8" % (K, N), flush=True)
    rng = np.random.default_rng(23)
    gen = torch.Generator(device="cuda:0").manual_seed(23)
    codes = torch.randint(-128, 128, (M, K), generator=gen, device="cuda:0", dtype=torch.int8)
    xs = torch.rand(M, generator=gen, device="cuda:0", dtype=torch.float32) * 0.01 + 1e-3
    Wp = _VALID[rng.integers(0, len(_VALID), size=(N, K // 4), dtype=np.uint8)]
    alpha = np.array([0.0211], np.float32)
    Y = hbl.hbl_gemm(codes, xs, 8, K, to_dev(Wp), to_dev(alpha), N, y_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), M - 8 + np.arange(8), rng.choice(M, 48, replace=False)]))
    ri = torch.from_numpy(rows).to("cuda:0")
    q = to_host(codes.index_select(0, ri))
    d = to_host(xs.index_select(0, ri))
    y_ref = oracle.rescale(oracle.int_gemm(q, oracle.unpack_ternary(Wp, K)), d, alpha[0])
    assert np.array_equal(to_host(Y.index_select(0, ri)), oracle.f32_to_bf16(y_ref))


def test_quantize_activations_past_2gib():
    """hbl_quantize_activations over 2^23 + 5 rows of K = 256 fp32 (8 GiB of
    input, so row offsets pass 2^31 bytes): codes and scales of sampled rows,
    the first and last 8 included, against the oracle (a code may differ only
    at a rounding boundary, checked)."""
    import torch
    M, K = (1 << 23) + 5, 256
    print("[case] quantize activations M=2^23+5 K=%d fp32" % K, flush=True)
    rng = np.random.default_rng(5)
    gen = torch.Generator(device="cuda:0").manual_seed(5)
    X = torch.randn((M, K), generator=gen, device="cuda:0", dtype=torch.float32)
    cfg = hbl.Config(act_bits=8)
    codes, xs, _, _ = hbl.hbl_quantize_activations(X, cfg)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), M - 8 + np.arange(8), rng.choice(M, 48, replace=False)]))
    ri = torch.from_numpy(rows).to("cuda:0")
    Xs = to_host(X.index_select(0, ri))
    ref = oracle.quantize_activations(Xs, bits=8, hadamard=cfg.hadamard)
    from parity import check_codes_end_to_end
    check_codes_end_to_end(unpack_codes(to_host(codes.index_select(0, ri)), K, 8), ref["z"], ref["s"], ref["q"],
                           "codes past 2 GiB")
    assert np.allclose(to_host(xs.index_select(0, ri)), ref["d"], rtol=1e-5, atol=0)
