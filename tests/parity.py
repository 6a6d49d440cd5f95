"""Parity helpers shared by the GPU tests: move seeded host arrays to the device,
call the library through its binding, and compare against the CPU oracle with
the tolerances the layer's contract states:

  * Hadamard output z: |z - z_ref| <= 1e-5 * max_k |z_ref| per row (fp32).
  * Quantised codes: bit-exact when the oracle quantises the GPU's own z with
    the GPU's own multiplier s ("identical quantiser inputs"); end to end, a
    code may differ (by exactly 1) only where the oracle's pre-round value
    z_ref*s_ref lies within 1e-5 (relative to the row's largest) of a
    rounding boundary.
  * Packed weights, int32 accumulators: bit-exact.
  * Final outputs: |y - y_ref| <= 1e-3 * max(|y_ref|, rms of y_ref's row).
"""
from __future__ import annotations

import numpy as np

import oracle

Z_TOL = 1e-5
BOUNDARY_TOL = 1e-5
Y_TOL = 1e-3


def torch():
    import torch as t
    return t


def to_dev(a: np.ndarray):
    """Host array -> device tensor; uint16 arrays are bf16 bit patterns."""
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(a.view(np.int16).copy()).view(t.bfloat16).to("cuda:0")
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def to_host(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.bfloat16:
        return x.view(t.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def unpack_codes(codes: np.ndarray, K: int, bits: int) -> np.ndarray:
    return codes.astype(np.int8) if bits == 8 else oracle.unpack_int4(codes, K)


def fp4_library_order(w4_rows: np.ndarray) -> np.ndarray:
    """Row-major FP4 bytes [N][K/2] (the oracle's O14 order: weight k of row n
    in byte k/2, low nibble for even k) rearranged into the library's W4 byte
    order as include/hbl.h defines it: bands of 256 rows; in a band of R rows
    the 64 bytes of K step s of every row form one block of R*64 bytes, row r
    at 64r, and the 16 bytes of weights 32c .. 32c+31 sit at 16*(c ^ ((r >> 2)
    & 3)).  Returns the N*K/2 bytes, flat."""
    N, KB = w4_rows.shape
    S = KB // 64
    out = np.empty(N * KB, dtype=np.uint8)
    for b0 in range(0, N, 256):
        R = min(256, N - b0)
        blk = w4_rows[b0:b0 + R].reshape(R, S, 4, 16)          # [r][s][chunk c][byte]
        r = np.arange(R)
        src = np.arange(4)[None, :] ^ ((r[:, None] >> 2) & 3)  # position p holds chunk p ^ f(r)
        phys = blk[r[:, None], :, src]                          # [r][p][s][byte]
        out[b0 * KB:(b0 + R) * KB] = phys.transpose(2, 0, 1, 3).reshape(-1)
    return out


def check_z(z_gpu: np.ndarray, z_ref: np.ndarray, what=""):
    for m in range(z_ref.shape[0]):
        scale = float(np.max(np.abs(z_ref[m])))
        err = float(np.max(np.abs(z_gpu[m].astype(np.float64) - z_ref[m])))
        assert err <= Z_TOL * max(scale, 1e-30), "%s row %d: |dz| %.3g > %.1g * %.3g" % (what, m, err, Z_TOL, scale)


def check_codes_given_inputs(z_gpu, s_gpu, d_gpu, q_gpu, bits, a4_mode, quant_eps, what=""):
    """Oracle O7/O8 on the GPU's own z: s and d equal (1 ulp for the absmean
    sum, whose fp64 order differs), codes bit-exact with the GPU's s."""
    for m in range(z_gpu.shape[0]):
        s_ref, d_ref = oracle.act_scale(z_gpu[m], bits, a4_mode=a4_mode, eps=quant_eps)
        ulps = 1 if (bits == 4 and a4_mode == oracle.A4_ABSMEAN) else 0
        for got, ref, name in ((s_gpu[m], s_ref, "s"), (d_gpu[m], d_ref, "d")):
            gap = abs(int(np.float32(got).view(np.int32)) - int(np.float32(ref).view(np.int32)))
            assert gap <= ulps, "%s row %d: %s %r vs oracle %r" % (what, m, name, got, ref)
        q_ref = oracle.act_codes(z_gpu[m], bits, s_gpu[m])
        bad = np.nonzero(q_ref != q_gpu[m])[0]
        assert bad.size == 0, "%s row %d: %d codes differ, first k=%d gpu %d oracle %d" % (
            what, m, bad.size, bad[0], q_gpu[m][bad[0]], q_ref[bad[0]])


def check_codes_end_to_end(q_gpu, z_ref, s_ref, q_ref, what=""):
    """Codes may differ from the oracle's only at rounding boundaries, by 1."""
    diff = q_gpu.astype(np.int32) - q_ref.astype(np.int32)
    rows, cols = np.nonzero(diff)
    if rows.size == 0:
        return 0
    assert np.all(np.abs(diff[rows, cols]) == 1), "%s: a code differs by more than 1" % what
    t = z_ref[rows, cols].astype(np.float64) * s_ref[rows].astype(np.float64)
    tmax = np.max(np.abs(z_ref[rows].astype(np.float64)), axis=1) * s_ref[rows].astype(np.float64)
    dist = np.abs(np.abs(t - np.floor(t)) - 0.5)
    assert np.all(dist <= BOUNDARY_TOL * np.maximum(tmax, 1.0)), \
        "%s: %d codes differ away from a rounding boundary (max dist %.3g)" % (what, rows.size, dist.max())
    return int(rows.size)


def bf16_ulp(r: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values at |r| (8 significant bits)."""
    e = np.floor(np.log2(np.maximum(np.abs(r), 1e-38)))
    return np.exp2(e - 7)


def check_y(y_gpu, y_ref, what="", bf16_out=False):
    """Output tolerance; a bf16 output also carries its own rounding (one bf16 ulp)."""
    y = y_gpu.astype(np.float64)
    r = y_ref.astype(np.float64)
    rms = np.sqrt(np.mean(r * r, axis=1, keepdims=True))
    tol = Y_TOL * np.maximum(np.abs(r), rms)
    if bf16_out:
        tol = tol + bf16_ulp(r)
    bad = np.abs(y - r) > tol
    assert not bad.any(), "%s: %d outputs outside 1e-3 (first %s: %r vs %r)" % (
        what, int(bad.sum()), tuple(np.argwhere(bad)[0]), y[tuple(np.argwhere(bad)[0])], r[tuple(np.argwhere(bad)[0])])


def y_to_f32(y: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f32(y) if y.dtype == np.uint16 else y


def dw_tolerance(M: int) -> float:
    """Relative bound (of sum_m |P_m q_mk|) for one weight-gradient element
    over M tokens, derived from the arithmetic:
      * P = fp32(dY * d) (2^-24) enters the products as a bf16 high part plus a
        bf16 remainder (unit roundoff 2^-8 each), so P is carried to 2^-16;
      * the products with the exact integer codes are exact in fp32, and the
        contraction runs over the high parts and then the remainders (2M
        terms) in matrix-core instructions of 16 products each, one fp32
        rounding per instruction into the accumulator: ceil(2M/16) roundings
        of at most 2^-24 of the running absolute sum.
    Never below 2^-15, the bound used for small M where the split dominates."""
    return max(2.0 ** -15, 2.0 ** -16 + 2.0 ** -24 + -(-2 * M // 16) * 2.0 ** -24)


def check_dw(got, dY, q, d, dW_ref, what=""):
    """Weight-gradient tolerance: each element within dw_tolerance(M) of the
    absolute sum of its terms, sum_m |P_m q_mk|.  (A bound relative to the
    row's largest value is wrong when a few tokens' terms cancel.)"""
    P = np.abs(oracle.as_f32(dY).astype(np.float64) * np.asarray(d, np.float64)[:, None])
    absum = P.T @ np.abs(np.asarray(q, np.float64))
    err = np.abs(np.asarray(got, np.float64) - dW_ref)
    tol = dw_tolerance(P.shape[0])
    bad = err > tol * absum + 1e-30
    assert not np.any(bad), "%s: %d elements beyond %.3g of sum|P q|, worst ratio %.3g" % (
        what, int(bad.sum()), tol, float(np.max(err / np.maximum(absum, 1e-30))))
