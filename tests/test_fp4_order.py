"""The W4 byte order that the GPU tests expect from hbl_pack_fp4
(parity.fp4_library_order) against the definition in include/hbl.h, written
out weight by weight: bands of 256 rows, K-step blocks of R*64 bytes, row r at
64r, the 16 bytes of weights 32c .. 32c+31 at 16*(c ^ ((r >> 2) & 3)), weight
k in the nibble k % 2 of its byte."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from parity import fp4_library_order  # noqa: E402


def _by_definition(w4_rows: np.ndarray) -> np.ndarray:
    N, KB = w4_rows.shape
    K = 2 * KB
    out = np.zeros(N * KB, dtype=np.uint8)
    for n in range(N):
        b = n // 256
        R = min(256, N - 256 * b)
        r = n - 256 * b
        for k in range(0, K, 2):   # weights k and k + 1 share a byte
            s, c = k // 128, (k % 128) // 32
            out[256 * b * KB + 64 * s * R + 64 * r + 16 * (c ^ ((r >> 2) & 3)) + (k % 32) // 2] = w4_rows[n, k // 2]
    return out


@pytest.mark.parametrize("N,K", [(4, 128), (8, 256), (300, 512), (512, 384), (257, 128)])
def test_fp4_library_order_matches_the_definition(N, K):
    w = np.random.default_rng(N * 7 + K).integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    assert np.array_equal(fp4_library_order(w), _by_definition(w))


def test_fp4_library_order_is_a_permutation_that_moves_chunks():
    w = np.arange(8 * 64, dtype=np.int64).reshape(8, 64).astype(np.uint8)   # K = 128: one step
    out = fp4_library_order(w)
    assert sorted(out.tolist()) == sorted(w.reshape(-1).tolist())
    assert np.array_equal(out[:4 * 64], w[:4].reshape(-1))                 # rows 0-3: chunks in place
    assert np.array_equal(out[4 * 64:4 * 64 + 16], w[4, 16:32])            # row 4: chunk 1 first
