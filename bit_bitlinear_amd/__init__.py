"""Python binding of libhbl.so, the H-BitLinear forward pass on MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the stream (the
current torch stream is passed to the library as its hipStream_t).  The
functions keep the C names of ``include/hbl.h``.

If the library is missing or fails to load, every call raises
``HblLibraryError``; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

__all__ = [
    "HblError", "HblLibraryError", "Config", "load_library", "declared_symbols",
    "hbl_packed_weight_bytes", "hbl_weight_workspace_bytes", "hbl_quantize_weights",
    "hbl_workspace_bytes", "hbl_forward_workspace_bytes", "hbl_quantize_activations", "hbl_gemm", "hbl_forward", "hbl_forward_latent",
    "hbl_quantize_heads", "hbl_backward_workspace_bytes", "hbl_backward", "hbl_status_string",
    "hbl_last_hip_error", "hbl_base3_weight_bytes", "hbl_pack_base3", "hbl_gemm_base3", "hbl_forward_base3",
    "hbl_fp4_weight_bytes", "hbl_pack_fp4", "hbl_fp6_codes_bytes", "hbl_quantize_activations_fp6",
    "hbl_gemm_fp6fp4", "hbl_forward_fp4_workspace_bytes", "hbl_forward_fp4", "hbl_forward_noalloc",
    "HBL_NOALLOC_SCRATCH_BYTES",
    "HBL_F32", "HBL_BF16", "HBL_NORM_RMS", "HBL_NORM_LN", "HBL_NORM_NONE",
    "HBL_A4_ABSMEAN_SQRT7", "HBL_A4_ABSMAX_7",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhbl.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "hbl.h")

HBL_F32, HBL_BF16 = 0, 1
HBL_NORM_RMS, HBL_NORM_LN, HBL_NORM_NONE = 0, 1, 2
HBL_A4_ABSMEAN_SQRT7, HBL_A4_ABSMAX_7 = 0, 1
HBL_OK = 0
HBL_NOALLOC_SCRATCH_BYTES = 32 << 20   # the static workspace of hbl_forward_noalloc

_STATUS_NAMES = {0: "HBL_OK", 1: "HBL_ERR_NULL", 2: "HBL_ERR_SHAPE", 3: "HBL_ERR_NOT_POW2", 4: "HBL_ERR_ALIGN",
                 5: "HBL_ERR_DTYPE", 6: "HBL_ERR_BITS", 7: "HBL_ERR_WORKSPACE", 8: "HBL_ERR_UNSUPPORTED",
                 9: "HBL_ERR_HIP"}


class HblLibraryError(RuntimeError):
    """libhbl.so is missing or cannot be loaded."""


class HblError(RuntimeError):
    """A library call returned a status other than HBL_OK."""

    def __init__(self, func, status, detail=""):
        self.func, self.status = func, status
        super().__init__("%s -> %s (%s)%s" % (func, _STATUS_NAMES.get(status, status),
                                              hbl_status_string(status), detail))


class _CConfig(ctypes.Structure):
    _fields_ = [("act_bits", ctypes.c_int32), ("hadamard", ctypes.c_int32), ("norm", ctypes.c_int32),
                ("a4_mode", ctypes.c_int32), ("norm_eps", ctypes.c_float), ("quant_eps", ctypes.c_float)]


class Config:
    """Layer configuration (mirrors hbl_config)."""

    def __init__(self, act_bits=8, hadamard=True, norm=HBL_NORM_RMS, a4_mode=HBL_A4_ABSMEAN_SQRT7,
                 norm_eps=1e-5, quant_eps=1e-5):
        self.act_bits, self.hadamard, self.norm, self.a4_mode = int(act_bits), bool(hadamard), int(norm), int(a4_mode)
        self.norm_eps, self.quant_eps = float(norm_eps), float(quant_eps)

    def c(self):
        return _CConfig(self.act_bits, int(self.hadamard), self.norm, self.a4_mode, self.norm_eps, self.quant_eps)

    def __repr__(self):
        return "Config(act_bits=%d, hadamard=%s, norm=%d, a4_mode=%d, norm_eps=%g, quant_eps=%g)" % (
            self.act_bits, self.hadamard, self.norm, self.a4_mode, self.norm_eps, self.quant_eps)


_lib = None


def load_library(path: str | None = None):
    """Load libhbl.so (once).  Raises HblLibraryError if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise HblLibraryError("libhbl.so not found at %s; build it with __graft_entry__.build() "
                              "(hipcc for gfx950)" % p)
    try:
        lib = ctypes.CDLL(p)
    except OSError as e:
        raise HblLibraryError("cannot load %s: %s" % (p, e)) from e
    P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    PSZ = ctypes.POINTER(ctypes.c_size_t)
    PCFG = ctypes.POINTER(_CConfig)
    sigs = {
        "hbl_packed_weight_bytes": [I64, I64, PSZ],
        "hbl_weight_workspace_bytes": [I64, I64, PSZ],
        "hbl_quantize_weights": [P, I32, I64, I64, F, P, P, P, SZ, P],
        "hbl_workspace_bytes": [I64, I64, PCFG, PSZ],
        "hbl_forward_workspace_bytes": [I64, I64, I64, PCFG, PSZ],
        "hbl_quantize_heads": [P, I32, I64, I64, I64, I32, F, P, P, P],
        "hbl_backward_workspace_bytes": [I64, I64, I64, PCFG, I32, PSZ],
        "hbl_backward": [P, I32, P, I32, I64, I64, P, P, P, I64, PCFG, P, P, P, SZ, P],
        "hbl_quantize_activations": [P, I32, I64, I64, P, PCFG, P, P, P, P, P],
        "hbl_gemm": [P, P, I32, I64, I64, P, P, I64, P, I32, P],
        "hbl_forward": [P, I32, I64, I64, P, P, P, I64, PCFG, P, I32, P, SZ, P],
        "hbl_forward_latent": [P, I32, I64, I64, P, P, I32, I64, F, PCFG, P, P, P, I32, P, SZ, P, SZ, P],
        "hbl_base3_weight_bytes": [I64, I64, PSZ],
        "hbl_pack_base3": [P, I64, I64, P, P],
        "hbl_gemm_base3": [P, P, I32, I64, I64, P, P, I64, P, I32, P],
        "hbl_forward_base3": [P, I32, I64, I64, P, P, P, I64, PCFG, P, I32, P, SZ, P],
        "hbl_fp4_weight_bytes": [I64, I64, PSZ],
        "hbl_pack_fp4": [P, I64, I64, P, P],
        "hbl_fp6_codes_bytes": [I64, I64, PSZ],
        "hbl_quantize_activations_fp6": [P, I32, I64, I64, P, PCFG, P, P, P],
        "hbl_gemm_fp6fp4": [P, P, I64, I64, P, P, I64, P, I32, P],
        "hbl_forward_fp4_workspace_bytes": [I64, I64, PCFG, PSZ],
        "hbl_forward_fp4": [P, I32, I64, I64, P, P, P, I64, PCFG, P, I32, P, SZ, P],
        "hbl_forward_noalloc": [P, I32, I64, I64, P, P, P, I64, PCFG, P, I32, P],
    }
    for name, argtypes in sigs.items():
        f = getattr(lib, name)
        f.argtypes = argtypes
        f.restype = ctypes.c_int
    lib.hbl_status_string.argtypes = [ctypes.c_int]
    lib.hbl_status_string.restype = ctypes.c_char_p
    lib.hbl_last_hip_error.argtypes = []
    lib.hbl_last_hip_error.restype = ctypes.c_int32
    if path is None:
        _lib = lib
    return lib


def declared_symbols(header: str = HEADER_PATH):
    """Names of the functions that include/hbl.h declares."""
    with open(header) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(hbl_\w+)\s*\(", text, re.M)))


def hbl_status_string(status: int) -> str:
    return load_library().hbl_status_string(int(status)).decode()


def hbl_last_hip_error() -> int:
    return int(load_library().hbl_last_hip_error())


# ------------------------------------------------------------------ helpers --
def _torch():
    import torch
    return torch


def _check(func, status):
    if status != HBL_OK:
        detail = ""
        if status == 9:
            detail = " hip error %d" % hbl_last_hip_error()
        raise HblError(func, status, detail)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.float32:
        return HBL_F32
    if t.dtype == torch.bfloat16:
        return HBL_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


def _torch_dtype(code):
    torch = _torch()
    return {HBL_F32: torch.float32, HBL_BF16: torch.bfloat16}[code]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _fits(t, nbytes, name):
    """The C ABI takes bare pointers, so every buffer's size is checked here:
    a buffer smaller than its shape needs would be written out of bounds."""
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError("%s holds %d bytes, the call needs %d" % (name, t.numel() * t.element_size(), nbytes))


def _esize(t):
    return 2 if t.dtype == _torch().bfloat16 else 4


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _size_out(func, *args):
    out = ctypes.c_size_t(0)
    _check(func.__name__, func(*args, ctypes.byref(out)))
    return int(out.value)


# -------------------------------------------------------------- entry points --
def hbl_packed_weight_bytes(N: int, K: int) -> int:
    return _size_out(load_library().hbl_packed_weight_bytes, N, K)


def hbl_weight_workspace_bytes(N: int, K: int) -> int:
    return _size_out(load_library().hbl_weight_workspace_bytes, N, K)


def hbl_forward_workspace_bytes(M: int, K: int, N: int, cfg: Config) -> int:
    """Workspace for the fastest hbl_forward / hbl_forward_latent path of an M x K by N x K layer."""
    c = cfg.c()
    return _size_out(load_library().hbl_forward_workspace_bytes, M, K, N, ctypes.byref(c))


def hbl_workspace_bytes(M: int, K: int, cfg: Config) -> int:
    c = cfg.c()
    return _size_out(load_library().hbl_workspace_bytes, M, K, ctypes.byref(c))


def hbl_quantize_weights(W, eps: float = 1e-5, W_packed=None, alpha=None, ws=None, stream=None):
    """Ternarise latent weights W [N][K] (float32/bfloat16, device).
    Returns (W_packed uint8 [N][K/4], alpha float32 [1]), both on W's device."""
    torch = _torch()
    lib = load_library()
    _dev(W, "W")
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=W.device)
    if ws is None:
        ws = torch.empty(hbl_weight_workspace_bytes(N, K), dtype=torch.uint8, device=W.device)
    _dev(W_packed, "W_packed"); _dev(alpha, "alpha"); _dev(ws, "ws")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha")
    _check("hbl_quantize_weights", lib.hbl_quantize_weights(_ptr(W), _dtype_code(W), N, K, float(eps), _ptr(W_packed),
                                                            _ptr(alpha), _ptr(ws), ws.numel() * ws.element_size(),
                                                            _stream(stream)))
    return W_packed, alpha


def hbl_quantize_activations(X, cfg: Config, gain=None, codes=None, xscale=None, z_debug=False, s_debug=False,
                             stream=None):
    """Norm + Hadamard + per-token quantisation of X [M][K].
    Returns (codes, xscale, z or None, s or None)."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(gain, "gain")
    M, K = X.shape
    if codes is None:
        shape = (M, K) if cfg.act_bits == 8 else (M, K // 2)
        codes = torch.empty(shape, dtype=torch.int8 if cfg.act_bits == 8 else torch.uint8, device=X.device)
    if xscale is None:
        xscale = torch.empty(M, dtype=torch.float32, device=X.device)
    z = torch.empty((M, K), dtype=torch.float32, device=X.device) if z_debug else None
    s = torch.empty(M, dtype=torch.float32, device=X.device) if s_debug else None
    _dev(codes, "codes"); _dev(xscale, "xscale")
    _fits(codes, M * K * cfg.act_bits // 8, "codes"); _fits(xscale, 4 * M, "xscale"); _fits(gain, 4 * K, "gain")
    c = cfg.c()
    _check("hbl_quantize_activations",
           lib.hbl_quantize_activations(_ptr(X), _dtype_code(X), M, K, _ptr(gain), ctypes.byref(c), _ptr(codes),
                                        _ptr(xscale), _ptr(z), _ptr(s), _stream(stream)))
    return codes, xscale, z, s


def hbl_gemm(codes, xscale, act_bits: int, K: int, W_packed, alpha, N: int, y_dtype=None, Y=None, stream=None):
    """Integer GEMM of activation codes against packed ternary weights with the
    rescale epilogue.  Returns Y [M][N] (float32 unless y_dtype says bfloat16)."""
    torch = _torch()
    lib = load_library()
    for t, n in ((codes, "codes"), (xscale, "xscale"), (W_packed, "W_packed"), (alpha, "alpha")):
        _dev(t, n)
    M = codes.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or torch.float32, device=codes.device)
    _dev(Y, "Y")
    _fits(codes, M * K * int(act_bits) // 8, "codes"); _fits(xscale, 4 * M, "xscale")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha"); _fits(Y, M * N * _esize(Y), "Y")
    _check("hbl_gemm", lib.hbl_gemm(_ptr(codes), _ptr(xscale), int(act_bits), M, K, _ptr(W_packed), _ptr(alpha), N,
                                    _ptr(Y), _dtype_code(Y), _stream(stream)))
    return Y


def hbl_forward(X, W_packed, alpha, N: int, cfg: Config, y_dtype=None, gain=None, Y=None, ws=None, stream=None):
    """The whole H-BitLinear forward of X [M][K] against packed weights.  Returns Y [M][N]."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(W_packed, "W_packed"); _dev(alpha, "alpha"); _dev(gain, "gain")
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, hbl_forward_workspace_bytes(M, K, N, cfg)), dtype=torch.uint8, device=X.device)
    _dev(Y, "Y"); _dev(ws, "ws")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(Y, M * N * _esize(Y), "Y")
    c = cfg.c()
    _check("hbl_forward", lib.hbl_forward(_ptr(X), _dtype_code(X), M, K, _ptr(gain), _ptr(W_packed), _ptr(alpha), N,
                                          ctypes.byref(c), _ptr(Y), _dtype_code(Y), _ptr(ws),
                                          ws.numel() * ws.element_size(), _stream(stream)))
    return Y


def hbl_forward_latent(X, W, cfg: Config, eps: float = 1e-5, y_dtype=None, gain=None, W_packed=None, alpha=None,
                       Y=None, ws=None, wws=None, stream=None):
    """Ternarise latent weights W [N][K] and run the forward of X [M][K] with
    them (hbl_quantize_weights + hbl_forward, fused to three launches).
    Returns (Y [M][N], W_packed uint8 [N][K/4], alpha float32 [1])."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(W, "W"); _dev(gain, "gain")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W has %d columns, X has %d" % (W.shape[1], K))
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=W.device)
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, hbl_forward_workspace_bytes(M, K, N, cfg)), dtype=torch.uint8, device=X.device)
    if wws is None:
        wws = torch.empty(hbl_weight_workspace_bytes(N, K), dtype=torch.uint8, device=W.device)
    for t, n in ((W_packed, "W_packed"), (alpha, "alpha"), (Y, "Y"), (ws, "ws"), (wws, "wws")):
        _dev(t, n)
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(Y, M * N * _esize(Y), "Y")
    c = cfg.c()
    _check("hbl_forward_latent", lib.hbl_forward_latent(
        _ptr(X), _dtype_code(X), M, K, _ptr(gain), _ptr(W), _dtype_code(W), N, float(eps), ctypes.byref(c),
        _ptr(W_packed), _ptr(alpha), _ptr(Y), _dtype_code(Y), _ptr(ws), ws.numel() * ws.element_size(),
        _ptr(wws), wws.numel() * wws.element_size(), _stream(stream)))
    return Y, W_packed, alpha


def hbl_quantize_heads(X, H: int, bits: int, eps: float = 1e-5, codes=None, scales=None, stream=None):
    """Per-(token, head) absmax quantisation of attention states X [M][H][D]
    (or [M][H*D]) to unsigned bits-bit codes.  Returns (codes uint8
    [M][H][D*bits/8], scales float32 [M][H])."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X")
    M = X.shape[0]
    D = X[0].numel() // H if M > 0 else (X.shape[-1] if X.dim() == 3 else X.shape[1] // H)
    if codes is None:
        codes = torch.empty((M, H, D * bits // 8), dtype=torch.uint8, device=X.device)
    if scales is None:
        scales = torch.empty((M, H), dtype=torch.float32, device=X.device)
    _dev(codes, "codes"); _dev(scales, "scales")
    if X.numel() != M * H * D:
        raise ValueError("X holds %d values, not %d tokens x %d heads x %d" % (X.numel(), M, H, D))
    _fits(codes, M * H * D * int(bits) // 8, "codes"); _fits(scales, 4 * M * H, "scales")
    _check("hbl_quantize_heads", lib.hbl_quantize_heads(_ptr(X), _dtype_code(X), M, H, D, int(bits), float(eps),
                                                        _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


def hbl_backward_workspace_bytes(M: int, K: int, N: int, cfg: Config, with_dw: bool = True) -> int:
    c = cfg.c()
    return _size_out(load_library().hbl_backward_workspace_bytes, M, K, N, ctypes.byref(c), int(bool(with_dw)))


def hbl_backward(dY, X, W_packed, alpha, cfg: Config, gain=None, want_dW: bool = True, dX=None, dW=None, ws=None,
                 stream=None):
    """The layer's straight-through backward.  dY [M][N] and X [M][K] (fp32 or
    bf16), W_packed [N][K/4], alpha [1].  Returns (dX float32 [M][K], dW
    float32 [N][K] or None)."""
    torch = _torch()
    lib = load_library()
    for t, n in ((dY, "dY"), (X, "X"), (W_packed, "W_packed"), (alpha, "alpha"), (gain, "gain")):
        _dev(t, n)
    M, K = X.shape
    N = dY.shape[1]
    if dX is None:
        dX = torch.empty((M, K), dtype=torch.float32, device=X.device)
    if want_dW and dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=X.device)
    if not want_dW:
        dW = None
    if ws is None:
        ws = torch.empty(max(1, hbl_backward_workspace_bytes(M, K, N, cfg, want_dW)), dtype=torch.uint8,
                         device=X.device)
    for t, n in ((dX, "dX"), (dW, "dW"), (ws, "ws")):
        _dev(t, n)
        if n != "ws" and t is not None and t.dtype != torch.float32:
            raise TypeError("%s must be float32" % n)
    if dY.shape[0] != M:
        raise ValueError("dY has %d rows, X has %d" % (dY.shape[0], M))
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(dX, 4 * M * K, "dX"); _fits(dW, 4 * N * K, "dW")
    c = cfg.c()
    _check("hbl_backward", lib.hbl_backward(_ptr(dY), _dtype_code(dY), _ptr(X), _dtype_code(X), M, K, _ptr(gain),
                                            _ptr(W_packed), _ptr(alpha), N, ctypes.byref(c), _ptr(dX), _ptr(dW),
                                            _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return dX, dW


def hbl_base3_weight_bytes(N: int, K: int) -> int:
    return _size_out(load_library().hbl_base3_weight_bytes, N, K)


def hbl_pack_base3(W_packed, K: int, W3=None, stream=None):
    """2-bit packed ternary weights [N][K/4] -> base-3 storage uint8 [N][16*ceil(K/80)]."""
    torch = _torch()
    lib = load_library()
    _dev(W_packed, "W_packed")
    N = W_packed.shape[0]
    if W3 is None:
        W3 = torch.empty((N, hbl_base3_weight_bytes(1, K)), dtype=torch.uint8, device=W_packed.device)
    _dev(W3, "W3")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(W3, hbl_base3_weight_bytes(max(N, 1), K) if N else 0, "W3")
    _check("hbl_pack_base3", lib.hbl_pack_base3(_ptr(W_packed), N, K, _ptr(W3), _stream(stream)))
    return W3


def hbl_gemm_base3(codes, xscale, act_bits: int, K: int, W3, alpha, N: int, y_dtype=None, Y=None, stream=None):
    """hbl_gemm with base-3 weights (1 to 4 tokens).  Returns Y [M][N]."""
    torch = _torch()
    lib = load_library()
    for t, n in ((codes, "codes"), (xscale, "xscale"), (W3, "W3"), (alpha, "alpha")):
        _dev(t, n)
    M = codes.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or torch.float32, device=codes.device)
    _dev(Y, "Y")
    _fits(codes, M * K * int(act_bits) // 8, "codes"); _fits(xscale, 4 * M, "xscale")
    _fits(W3, N * hbl_base3_weight_bytes(1, K), "W3"); _fits(alpha, 4, "alpha"); _fits(Y, M * N * _esize(Y), "Y")
    _check("hbl_gemm_base3", lib.hbl_gemm_base3(_ptr(codes), _ptr(xscale), int(act_bits), M, K, _ptr(W3),
                                                _ptr(alpha), N, _ptr(Y), _dtype_code(Y), _stream(stream)))
    return Y


def hbl_forward_base3(X, W3, alpha, N: int, cfg: Config, y_dtype=None, gain=None, Y=None, ws=None, stream=None):
    """hbl_forward with base-3 weights (1 to 4 tokens).  Returns Y [M][N]."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(W3, "W3"); _dev(alpha, "alpha"); _dev(gain, "gain")
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, hbl_workspace_bytes(M, K, cfg)), dtype=torch.uint8, device=X.device)
    _dev(Y, "Y"); _dev(ws, "ws")
    _fits(W3, N * hbl_base3_weight_bytes(1, K), "W3"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(Y, M * N * _esize(Y), "Y")
    c = cfg.c()
    _check("hbl_forward_base3", lib.hbl_forward_base3(_ptr(X), _dtype_code(X), M, K, _ptr(gain), _ptr(W3),
                                                      _ptr(alpha), N, ctypes.byref(c), _ptr(Y), _dtype_code(Y),
                                                      _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return Y


# ------------------------------------------ FP4 weights and FP6 codes (INT4) --
def hbl_fp4_weight_bytes(N: int, K: int) -> int:
    return _size_out(load_library().hbl_fp4_weight_bytes, N, K)


def hbl_fp6_codes_bytes(M: int, K: int) -> int:
    return _size_out(load_library().hbl_fp6_codes_bytes, M, K)


def hbl_forward_fp4_workspace_bytes(M: int, K: int, cfg: Config) -> int:
    c = cfg.c()
    return _size_out(load_library().hbl_forward_fp4_workspace_bytes, M, K, ctypes.byref(c))


def hbl_pack_fp4(W_packed, K: int, W4=None, stream=None):
    """2-bit packed ternary weights [N][K/4] -> FP4 E2M1 weights, N*K/2 bytes
    (held as uint8 [N][K/2]) in the library's W4 order; K % 128 == 0."""
    torch = _torch()
    lib = load_library()
    _dev(W_packed, "W_packed")
    N = W_packed.shape[0]
    if W4 is None:
        W4 = torch.empty((N, K // 2), dtype=torch.uint8, device=W_packed.device)
    _dev(W4, "W4")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(W4, N * K // 2, "W4")
    _check("hbl_pack_fp4", lib.hbl_pack_fp4(_ptr(W_packed), N, K, _ptr(W4), _stream(stream)))
    return W4


def hbl_quantize_activations_fp6(X, cfg: Config, gain=None, codes6=None, xscale=None, stream=None):
    """INT4 activation codes of X [M][K] as FP6 (the FP6 x FP4 GEMM's operand
    order, private to the library, for these M and K).  Returns (codes6 uint8
    [M][K*3/4] as storage, xscale float32 [M])."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(gain, "gain")
    M, K = X.shape
    if codes6 is None:
        codes6 = torch.empty((M, K * 3 // 4), dtype=torch.uint8, device=X.device)
    if xscale is None:
        xscale = torch.empty(M, dtype=torch.float32, device=X.device)
    _dev(codes6, "codes6"); _dev(xscale, "xscale")
    _fits(codes6, M * K * 3 // 4, "codes6"); _fits(xscale, 4 * M, "xscale"); _fits(gain, 4 * K, "gain")
    c = cfg.c()
    _check("hbl_quantize_activations_fp6",
           lib.hbl_quantize_activations_fp6(_ptr(X), _dtype_code(X), M, K, _ptr(gain), ctypes.byref(c), _ptr(codes6),
                                            _ptr(xscale), _stream(stream)))
    return codes6, xscale


def hbl_gemm_fp6fp4(codes6, xscale, K: int, W4, alpha, N: int, y_dtype=None, Y=None, stream=None):
    """FP6 codes x FP4 weights on the FP6 x FP4 matrix cores with the rescale
    epilogue.  Returns Y [M][N]."""
    torch = _torch()
    lib = load_library()
    for t, n in ((codes6, "codes6"), (xscale, "xscale"), (W4, "W4"), (alpha, "alpha")):
        _dev(t, n)
    M = codes6.shape[0]
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or torch.float32, device=codes6.device)
    _dev(Y, "Y")
    _fits(codes6, M * K * 3 // 4, "codes6"); _fits(xscale, 4 * M, "xscale")
    _fits(W4, N * K // 2, "W4"); _fits(alpha, 4, "alpha"); _fits(Y, M * N * _esize(Y), "Y")
    _check("hbl_gemm_fp6fp4", lib.hbl_gemm_fp6fp4(_ptr(codes6), _ptr(xscale), M, K, _ptr(W4), _ptr(alpha), N,
                                                  _ptr(Y), _dtype_code(Y), _stream(stream)))
    return Y


def hbl_forward_fp4(X, W4, alpha, N: int, cfg: Config, y_dtype=None, gain=None, Y=None, ws=None, stream=None):
    """The INT4 forward of X [M][K] against FP4 weights (FP6 x FP4 matrix
    cores).  Bit for bit hbl_forward on the same ternary values.  Returns Y."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(W4, "W4"); _dev(alpha, "alpha"); _dev(gain, "gain")
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device)
    if ws is None:
        ws = torch.empty(max(1, hbl_forward_fp4_workspace_bytes(M, K, cfg)), dtype=torch.uint8, device=X.device)
    _dev(Y, "Y"); _dev(ws, "ws")
    _fits(W4, N * K // 2, "W4"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(Y, M * N * _esize(Y), "Y")
    c = cfg.c()
    _check("hbl_forward_fp4", lib.hbl_forward_fp4(_ptr(X), _dtype_code(X), M, K, _ptr(gain), _ptr(W4), _ptr(alpha),
                                                  N, ctypes.byref(c), _ptr(Y), _dtype_code(Y), _ptr(ws),
                                                  ws.numel() * ws.element_size(), _stream(stream)))
    return Y


def hbl_forward_noalloc(X, W_packed, alpha, N: int, cfg: Config, y_dtype=None, gain=None, Y=None, stream=None):
    """hbl_forward with the workspace in the library's static device array
    (no allocation by the library; Y is allocated here only when not given).
    Returns Y [M][N]."""
    torch = _torch()
    lib = load_library()
    _dev(X, "X"); _dev(W_packed, "W_packed"); _dev(alpha, "alpha"); _dev(gain, "gain")
    M, K = X.shape
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype or X.dtype, device=X.device)
    _dev(Y, "Y")
    _fits(W_packed, N * K // 4, "W_packed"); _fits(alpha, 4, "alpha"); _fits(gain, 4 * K, "gain")
    _fits(Y, M * N * _esize(Y), "Y")
    c = cfg.c()
    _check("hbl_forward_noalloc", lib.hbl_forward_noalloc(_ptr(X), _dtype_code(X), M, K, _ptr(gain), _ptr(W_packed),
                                                          _ptr(alpha), N, ctypes.byref(c), _ptr(Y), _dtype_code(Y),
                                                          _stream(stream)))
    return Y
