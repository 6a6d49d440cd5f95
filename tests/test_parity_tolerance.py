"""The GPU tests' weight-gradient tolerance (parity.check_dw), checked on the
CPU: it accepts dW computed the way the matrix cores compute it (dY*d split
into a bf16 high part and remainder, products summed in fp32) and rejects the
mistakes it is there to catch (dY*d in one bf16, a dropped token, a flipped
sign), including where the tokens' terms cancel and the result is small."""
import numpy as np
import pytest

import oracle
from parity import check_dw


def _bf16_round(x):
    """Round fp32 to the nearest bf16 (ties to even), returned as fp32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32)


def _case(M, K, N, seed):
    rng = np.random.default_rng(seed)
    dY = rng.standard_normal((M, N)).astype(np.float32)
    q = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    d = (rng.random(M).astype(np.float32) * np.float32(0.05) + np.float32(0.01)).astype(np.float32)
    return dY, q, d


def _split_f32_sum(dY, q, d):
    P = (dY * d[:, None]).astype(np.float32)
    hi = _bf16_round(P)
    lo = _bf16_round((P - hi).astype(np.float32))
    acc = np.zeros((dY.shape[1], q.shape[1]), np.float32)
    for m in range(dY.shape[0]):
        acc += np.outer(hi[m], q[m].astype(np.float32)).astype(np.float32)
        acc += np.outer(lo[m], q[m].astype(np.float32)).astype(np.float32)
    return acc


@pytest.mark.parametrize("M,seed", [(1, 0), (7, 1), (64, 2), (300, 3)])
def test_check_dw_accepts_split_bf16_with_f32_sums(M, seed):
    dY, q, d = _case(M, 40, 24, seed)
    check_dw(_split_f32_sum(dY, q, d), dY, q, d, oracle.weight_grad(dY, q, d), "split")


@pytest.mark.parametrize("M,seed", [(7, 1), (64, 2)])
def test_check_dw_rejects_single_bf16(M, seed):
    dY, q, d = _case(M, 40, 24, seed)
    P1 = _bf16_round((dY * d[:, None]).astype(np.float32))
    coarse = P1.astype(np.float64).T @ q.astype(np.float64)
    with pytest.raises(AssertionError):
        check_dw(coarse, dY, q, d, oracle.weight_grad(dY, q, d), "one bf16")


def test_check_dw_rejects_dropped_token_and_sign():
    dY, q, d = _case(7, 40, 24, 4)
    ref = oracle.weight_grad(dY, q, d)
    with pytest.raises(AssertionError):
        check_dw(oracle.weight_grad(dY[1:], q[1:], d[1:]), dY, q, d, ref, "dropped token")
    with pytest.raises(AssertionError):
        check_dw(-ref, dY, q, d, ref, "sign")


def test_check_dw_accepts_cancelling_terms():
    """Two tokens whose terms nearly cancel: the exact result is tiny, the
    split-bf16 error is not, and the bound (from the absolute sum) allows it."""
    rng = np.random.default_rng(5)
    N, K = 16, 32
    base = rng.standard_normal(N).astype(np.float32)
    dY = np.stack([base, -base * np.float32(1.0000001) + np.float32(1e-3)]).astype(np.float32)
    q = np.tile(rng.integers(1, 8, size=(1, K)).astype(np.int8), (2, 1))
    d = np.array([0.0371, 0.0371], np.float32)
    got = _split_f32_sum(dY, q, d)
    ref = oracle.weight_grad(dY, q, d)
    check_dw(got, dY, q, d, ref, "cancel")
