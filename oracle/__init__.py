"""CPU oracle for the H-BitLinear forward pass (BitNet v2) -- test infrastructure.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this package.  The HIP library never does; the two share no
code.  The arithmetic lives in ``hbl_oracle.c`` (plain C, fp64 where stated);
this module only builds it, loads it with ctypes and marshals numpy arrays.

Every function here returns fresh numpy arrays and takes host arrays:
  * ``X`` as float32 ``[M][K]`` or bf16 bit patterns (uint16) ``[M][K]``
  * latent weights ``W`` as float32 ``[N][K]`` (bf16 patterns are converted exactly)

Steps and the passages they follow are documented in ``hbl_oracle.c`` (O1-O10 for
the layer, O11 for the low-bit attention states beside it, O12 for the layer's
straight-through backward).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hbl_oracle.c")
_LIB = os.path.join(_HERE, "libhbl_oracle.so")

NORM_RMS, NORM_LN, NORM_NONE = 0, 1, 2
A4_ABSMEAN, A4_ABSMAX = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile hbl_oracle.c with gcc (no fast-math, no fp contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # HBL_ORACLE_SO points at another build of an oracle source; the mutation
    # test uses it to run the pins against deliberately broken copies.
    path = os.environ.get("HBL_ORACLE_SO")
    if not path:
        path = _LIB
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    I = ctypes.c_int
    lib.hbo_num_threads.restype = I
    lib.hbo_set_num_threads.argtypes = [I]
    lib.hbo_bf16_to_f32.argtypes = [P, I64, P]
    lib.hbo_f32_to_bf16.argtypes = [P, I64, P]
    lib.hbo_weight_alpha.argtypes = [P, I64]
    lib.hbo_weight_alpha.restype = F
    lib.hbo_ternarize.argtypes = [P, I64, F, F, P]
    lib.hbo_pack_ternary.argtypes = [P, I64, I64, P]
    lib.hbo_pack_ternary.restype = I
    lib.hbo_unpack_ternary.argtypes = [P, I64, I64, P]
    lib.hbo_unpack_ternary.restype = I
    lib.hbo_quantize_weights.argtypes = [P, I64, I64, F, P, P, P]
    lib.hbo_quantize_weights.restype = I
    lib.hbo_norm_row.argtypes = [P, I64, P, I, F, P]
    lib.hbo_hadamard_row.argtypes = [P, I64, P]
    lib.hbo_act_scale.argtypes = [P, I64, I, I, F, P, P]
    lib.hbo_act_scale.restype = I
    lib.hbo_act_codes.argtypes = [P, I64, I, F, P]
    lib.hbo_act_codes.restype = I
    lib.hbo_pack_int4.argtypes = [P, I64, I64, P]
    lib.hbo_pack_int4.restype = I
    lib.hbo_unpack_int4.argtypes = [P, I64, I64, P]
    lib.hbo_unpack_int4.restype = I
    lib.hbo_quantize_activations.argtypes = [P, I64, I64, P, I, F, I, I, I, F, P, P, P, P]
    lib.hbo_quantize_activations.restype = I
    lib.hbo_int_gemm.argtypes = [P, P, I64, I64, I64, P]
    lib.hbo_int_gemm.restype = I
    lib.hbo_rescale.argtypes = [P, P, F, I64, I64, P]
    lib.hbo_quantize_heads.argtypes = [P, I64, I64, I64, I, F, P, P]
    lib.hbo_quantize_heads.restype = I
    lib.hbo_unpack_heads.argtypes = [P, I64, I64, I, P]
    lib.hbo_unpack_heads.restype = I
    lib.hbo_backward.argtypes = [P, P, I64, I64, P, I, F, I, I, I, F, P, F, I64, P, P]
    lib.hbo_backward.restype = I
    lib.hbo_weight_grad.argtypes = [P, P, P, I64, I64, I64, P]
    lib.hbo_base3_row_bytes.argtypes = [I64]
    lib.hbo_base3_row_bytes.restype = I64
    lib.hbo_pack_base3.argtypes = [P, I64, I64, P]
    lib.hbo_pack_base3.restype = I
    lib.hbo_unpack_base3.argtypes = [P, I64, I64, P]
    lib.hbo_unpack_base3.restype = I
    lib.hbo_pack_fp4.argtypes = [P, I64, I64, P]
    lib.hbo_pack_fp4.restype = I
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s rejected its arguments" % what)


def num_threads() -> int:
    return int(_load().hbo_num_threads())


def set_num_threads(n: int) -> None:
    _load().hbo_set_num_threads(int(n))


# ---------------------------------------------------------------- O4 -------
def bf16_to_f32(x_bits: np.ndarray) -> np.ndarray:
    x = _c(x_bits, np.uint16)
    out = np.empty(x.shape, np.float32)
    _load().hbo_bf16_to_f32(_ptr(x), x.size, _ptr(out))
    return out


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().hbo_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def as_f32(X: np.ndarray) -> np.ndarray:
    """fp32 view of an input: fp32 passes through, bf16 bit patterns convert exactly."""
    if X.dtype == np.uint16:
        return bf16_to_f32(X)
    return _c(X, np.float32)


# ---------------------------------------------------------- O1-O3 ----------
def weight_alpha(W: np.ndarray) -> np.float32:
    W = as_f32(W)
    return np.float32(_load().hbo_weight_alpha(_ptr(W), W.size))


def ternarize(W: np.ndarray, alpha: float, eps: float) -> np.ndarray:
    W = as_f32(W)
    out = np.empty(W.shape, np.int8)
    _load().hbo_ternarize(_ptr(W), W.size, float(alpha), float(eps), _ptr(out))
    return out


def pack_ternary(Wq: np.ndarray) -> np.ndarray:
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    out = np.empty((N, K // 4), np.uint8)
    _check(_load().hbo_pack_ternary(_ptr(Wq), N, K, _ptr(out)), "pack_ternary")
    return out


def unpack_ternary(Wp: np.ndarray, K: int) -> np.ndarray:
    Wp = _c(Wp, np.uint8)
    N = Wp.shape[0]
    out = np.empty((N, K), np.int8)
    _check(_load().hbo_unpack_ternary(_ptr(Wp), N, K, _ptr(out)), "unpack_ternary")
    return out


def quantize_weights(W: np.ndarray, eps: float = 1e-5):
    """O1-O3: returns (Wq int8 [N][K], W_packed uint8 [N][K/4], alpha float32)."""
    W = as_f32(W)
    N, K = W.shape
    Wq = np.empty((N, K), np.int8)
    Wp = np.empty((N, K // 4), np.uint8)
    alpha = np.zeros(1, np.float32)
    _check(_load().hbo_quantize_weights(_ptr(W), N, K, float(eps), _ptr(Wq), _ptr(Wp), _ptr(alpha)),
           "quantize_weights")
    return Wq, Wp, alpha[0]


# ---------------------------------------------------------- O5, O6 ---------
def norm_rows(X: np.ndarray, gain=None, norm: int = NORM_RMS, eps: float = 1e-5) -> np.ndarray:
    """O5 on every row; fp64 result."""
    X = as_f32(X)
    M, K = X.shape
    g = None if gain is None else _c(gain, np.float32)
    out = np.empty((M, K), np.float64)
    lib = _load()
    for m in range(M):
        row = X[m]
        lib.hbo_norm_row(_ptr(row), K, _ptr(g), norm, float(eps), _ptr(out[m]))
    return out


def hadamard_rows(R: np.ndarray) -> np.ndarray:
    """O6 (dense normalised Sylvester) on every fp64 row; fp64 result."""
    R = _c(R, np.float64)
    if R.ndim == 1:
        R = R[None, :]
    M, K = R.shape
    out = np.empty((M, K), np.float64)
    lib = _load()
    for m in range(M):
        lib.hbo_hadamard_row(_ptr(R[m]), K, _ptr(out[m]))
    return out


# ---------------------------------------------------------- O7, O8 ---------
def act_scale(z: np.ndarray, bits: int, a4_mode: int = A4_ABSMEAN, eps: float = 1e-5):
    """O7 for one fp32 row: returns (s, d) as float32."""
    z = _c(z, np.float32).ravel()
    s = np.zeros(1, np.float32)
    d = np.zeros(1, np.float32)
    _check(_load().hbo_act_scale(_ptr(z), z.size, bits, a4_mode, float(eps), _ptr(s), _ptr(d)), "act_scale")
    return s[0], d[0]


def act_codes(z: np.ndarray, bits: int, s: float) -> np.ndarray:
    """O8 for one fp32 row with a given multiplier s: int8 codes."""
    z = _c(z, np.float32).ravel()
    q = np.empty(z.size, np.int8)
    _check(_load().hbo_act_codes(_ptr(z), z.size, bits, float(np.float32(s)), _ptr(q)), "act_codes")
    return q


def pack_int4(q: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    M, K = q.shape
    out = np.empty((M, K // 2), np.uint8)
    _check(_load().hbo_pack_int4(_ptr(q), M, K, _ptr(out)), "pack_int4")
    return out


def unpack_int4(p: np.ndarray, K: int) -> np.ndarray:
    p = _c(p, np.uint8)
    M = p.shape[0]
    out = np.empty((M, K), np.int8)
    _check(_load().hbo_unpack_int4(_ptr(p), M, K, _ptr(out)), "unpack_int4")
    return out


def quantize_activations(X: np.ndarray, *, bits: int, hadamard: bool = True, gain=None,
                         norm: int = NORM_RMS, norm_eps: float = 1e-5, quant_eps: float = 1e-5,
                         a4_mode: int = A4_ABSMEAN, want_z: bool = True):
    """O4-O8 on every row.  Returns dict(z fp32 [M][K] or None, q int8 [M][K], s, d float32 [M])."""
    X = as_f32(X)
    M, K = X.shape
    g = None if gain is None else _c(gain, np.float32)
    z = np.empty((M, K), np.float32) if want_z else None
    q = np.empty((M, K), np.int8)
    s = np.empty(M, np.float32)
    d = np.empty(M, np.float32)
    _check(_load().hbo_quantize_activations(_ptr(X), M, K, _ptr(g), norm, float(norm_eps), int(bool(hadamard)),
                                            bits, a4_mode, float(quant_eps), _ptr(z), _ptr(q), _ptr(s), _ptr(d)),
           "quantize_activations")
    return {"z": z, "q": q, "s": s, "d": d}


# ---------------------------------------------------------- O9, O10 --------
def int_gemm(q: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    q = _c(q, np.int8)
    Wq = _c(Wq, np.int8)
    M, K = q.shape
    N, K2 = Wq.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    acc = np.empty((M, N), np.int32)
    _check(_load().hbo_int_gemm(_ptr(q), _ptr(Wq), M, N, K, _ptr(acc)), "int_gemm (overflow)")
    return acc


def rescale(acc: np.ndarray, d: np.ndarray, alpha: float) -> np.ndarray:
    acc = _c(acc, np.int32)
    d = _c(d, np.float32)
    M, N = acc.shape
    y = np.empty((M, N), np.float32)
    _load().hbo_rescale(_ptr(acc), _ptr(d), float(np.float32(alpha)), M, N, _ptr(y))
    return y


def forward(X: np.ndarray, Wq: np.ndarray, alpha: float, *, bits: int, hadamard: bool = True, gain=None,
            norm: int = NORM_RMS, norm_eps: float = 1e-5, quant_eps: float = 1e-5, a4_mode: int = A4_ABSMEAN):
    """O4-O10: returns dict(y fp32 [M][N], acc int32, q int8, d, s, z)."""
    qa = quantize_activations(X, bits=bits, hadamard=hadamard, gain=gain, norm=norm, norm_eps=norm_eps,
                              quant_eps=quant_eps, a4_mode=a4_mode)
    acc = int_gemm(qa["q"], Wq)
    y = rescale(acc, qa["d"], alpha)
    qa.update({"acc": acc, "y": y})
    return qa


# ---------------------------------------------------------------- O11 ------
def quantize_heads(X: np.ndarray, bits: int, eps: float = 1e-5):
    """O11: X [M][H][D] (fp32, or bf16 bit patterns) -> (packed codes uint8
    [M][H][D*bits/8], dequant factors float32 [M][H])."""
    x = as_f32(X)
    if x.ndim != 3:
        raise ValueError("X must be [M][H][D]")
    M, H, D = x.shape
    x = _c(x, np.float32)
    codes = np.empty((M, H, D * bits // 8), np.uint8)
    d = np.empty((M, H), np.float32)
    _check(_load().hbo_quantize_heads(_ptr(x), M, H, D, int(bits), float(np.float32(eps)), _ptr(codes), _ptr(d)),
           "quantize_heads")
    return codes, d


def unpack_heads(codes: np.ndarray, D: int, bits: int) -> np.ndarray:
    """Packed head codes [..][D*bits/8] -> one uint8 code per element [..][D]."""
    c = _c(codes, np.uint8)
    lead = c.shape[:-1]
    V = int(np.prod(lead)) if lead else 1
    u = np.empty(lead + (D,), np.uint8)
    _check(_load().hbo_unpack_heads(_ptr(c), V, D, int(bits), _ptr(u)), "unpack_heads")
    return u


# ---------------------------------------------------------------- O12 ------
def backward(dY: np.ndarray, X: np.ndarray, Wq: np.ndarray, alpha: float, *, bits: int, hadamard: bool = True,
             gain=None, norm: int = NORM_RMS, norm_eps: float = 1e-5, quant_eps: float = 1e-5,
             a4_mode: int = A4_ABSMEAN, want_dW: bool = True):
    """O12: the straight-through backward.  dY [M][N] (fp32 or bf16 bit
    patterns), X [M][K] as for quantize_activations, Wq int8 [N][K].
    Returns (dX fp64 [M][K], dW fp64 [N][K] or None)."""
    dy = as_f32(dY)
    x = as_f32(X)
    M, K = x.shape
    N = Wq.shape[0]
    g = None if gain is None else _c(gain, np.float32)
    Wq = _c(Wq, np.int8)
    dX = np.empty((M, K), np.float64)
    dW = np.empty((N, K), np.float64) if want_dW else None
    _check(_load().hbo_backward(_ptr(_c(dy, np.float32)), _ptr(x), M, K, _ptr(g), int(norm), float(norm_eps),
                                int(bool(hadamard)), int(bits), int(a4_mode), float(quant_eps), _ptr(Wq),
                                float(np.float32(alpha)), N, _ptr(dX), _ptr(dW)), "backward")
    return dX, dW


def weight_grad(dY: np.ndarray, q: np.ndarray, d: np.ndarray) -> np.ndarray:
    """O12, weight part: dW = dY^T (d * q) in fp64 for given codes q int8
    [M][K] and factors d [M]; dY fp32 or bf16 bit patterns [M][N]."""
    dy = _c(as_f32(dY), np.float32)
    q = _c(q, np.int8)
    d = _c(d, np.float32)
    M, N = dy.shape
    K = q.shape[1]
    dW = np.empty((N, K), np.float64)
    _load().hbo_weight_grad(_ptr(dy), _ptr(q), _ptr(d), M, N, K, _ptr(dW))
    return dW


# ---------------------------------------------------------------- O13 ------
def base3_row_bytes(K: int) -> int:
    """Bytes per row of the base-3 weight format (16 * ceil(K / 80))."""
    return int(_load().hbo_base3_row_bytes(int(K)))


def pack_base3(Wq: np.ndarray) -> np.ndarray:
    """O13: ternary int8 [N][K] -> uint8 [N][base3_row_bytes(K)], five weights
    per byte as base-3 digits t + 1, the first weight least significant."""
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    out = np.empty((N, base3_row_bytes(K)), np.uint8)
    _check(_load().hbo_pack_base3(_ptr(Wq), N, K, _ptr(out)), "pack_base3")
    return out


def unpack_base3(W3: np.ndarray, K: int) -> np.ndarray:
    """The inverse of pack_base3 (rejects bytes above 242 and nonzero padding)."""
    W3 = _c(W3, np.uint8)
    N = W3.shape[0]
    if W3.shape[1] != base3_row_bytes(K):
        raise ValueError("row length does not match K")
    out = np.empty((N, K), np.int8)
    _check(_load().hbo_unpack_base3(_ptr(W3), N, K, _ptr(out)), "unpack_base3")
    return out


# ---------------------------------------------------------------- O14 ------
def pack_fp4(Wq: np.ndarray) -> np.ndarray:
    """O14: ternary int8 [N][K] -> FP4 E2M1 weights uint8 [N][K/2] (low nibble = even k)."""
    Wq = _c(Wq, np.int8)
    N, K = Wq.shape
    out = np.empty((N, K // 2), np.uint8)
    _check(_load().hbo_pack_fp4(_ptr(Wq), N, K, _ptr(out)), "pack_fp4")
    return out
