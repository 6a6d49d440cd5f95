"""CPU tests of the C ABI: the library loads, exports every function that
include/hbl.h declares, and rejects invalid arguments on the host before
anything is queued (these calls need no GPU)."""
import ctypes

import pytest

import bit_bitlinear_amd as hbl

# Fake, never-dereferenced device addresses (validation must reject first).
A16 = ctypes.c_void_p(0x10000)
A16b = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)


@pytest.fixture(scope="module")
def lib():
    return hbl.load_library()


def test_library_exports_every_declared_symbol(lib):
    names = hbl.declared_symbols()
    assert len(names) == 26
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(hbl.HblLibraryError):
        hbl.load_library(str(tmp_path / "libhbl.so"))


def test_status_strings(lib):
    for s in range(10):
        assert hbl.hbl_status_string(s)
    assert hbl.hbl_status_string(12345) == "unknown status"
    assert hbl.hbl_last_hip_error() == 0


def test_size_queries():
    assert hbl.hbl_packed_weight_bytes(256, 256) == 256 * 64
    assert hbl.hbl_packed_weight_bytes(4096, 16384) == 4096 * 4096
    assert hbl.hbl_weight_workspace_bytes(2048, 2048) >= 8
    ws8 = hbl.hbl_workspace_bytes(4096, 2048, hbl.Config(act_bits=8))
    ws4 = hbl.hbl_workspace_bytes(4096, 2048, hbl.Config(act_bits=4))
    assert ws8 >= 4096 * 2048 + 4096 * 4 and ws4 >= 4096 * 1024 + 4096 * 4 and ws4 < ws8
    assert hbl.hbl_workspace_bytes(0, 2048, hbl.Config()) == 0
    # up to 64 tokens the codes region holds whole 16-row tiles
    assert hbl.hbl_workspace_bytes(5, 1024, hbl.Config(act_bits=8)) >= 16 * 1024 + 5 * 4
    assert hbl.hbl_workspace_bytes(65, 1024, hbl.Config(act_bits=8)) < 80 * 1024
    # the FP6 x FP4 path's workspace: INT4 prefill shapes only
    c4, c8 = hbl.Config(act_bits=4), hbl.Config(act_bits=8)
    big = hbl.hbl_forward_workspace_bytes(8192, 16384, 4096, c4)
    assert big >= 8192 * 16384 * 3 // 4 + 8192 * 4 + 4096 * 16384 // 2
    assert hbl.hbl_forward_workspace_bytes(8192, 16384, 4096, c8) == hbl.hbl_workspace_bytes(8192, 16384, c8)
    assert hbl.hbl_forward_workspace_bytes(64, 8192, 4096, c4) == hbl.hbl_workspace_bytes(64, 8192, c4)
    assert hbl.hbl_forward_workspace_bytes(256, 4096, 4096, c4) == hbl.hbl_workspace_bytes(256, 4096, c4)
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_forward_workspace_bytes(8, 256, 0, c4)
    assert e.value.status == 2
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_packed_weight_bytes(16, 40)
    assert e.value.status == 4
    with pytest.raises(hbl.HblError):
        hbl.hbl_workspace_bytes(8, 256, hbl.Config(act_bits=5))


def _act(lib, X=A16, dt=0, M=8, K=256, gain=None, cfg=None, codes=A16b, xs=A16b, z=None, s=None):
    c = (cfg or hbl.Config()).c()
    return lib.hbl_quantize_activations(X, dt, M, K, gain, ctypes.byref(c), codes, xs, z, s, None)


def test_quantize_activations_validation(lib):
    assert _act(lib, K=300) == 3                                   # not a power of two
    assert _act(lib, K=128) == 2 and _act(lib, K=65536) == 2       # outside [256, 32768]
    assert _act(lib, M=-1) == 2
    assert _act(lib, dt=7) == 5
    assert _act(lib, cfg=hbl.Config(act_bits=5)) == 6
    assert _act(lib, cfg=hbl.Config(act_bits=4, a4_mode=9)) == 6
    assert _act(lib, cfg=hbl.Config(norm=7)) == 6
    assert _act(lib, cfg=hbl.Config(norm_eps=-1.0)) == 2
    assert _act(lib, X=None) == 1 and _act(lib, codes=None) == 1 and _act(lib, xs=None) == 1
    assert _act(lib, X=MIS) == 4 and _act(lib, z=MIS) == 4
    assert _act(lib, M=0, X=None) == 0                              # empty input: nothing queued
    c = hbl.Config().c()
    assert lib.hbl_quantize_activations(A16, 0, 8, 256, None, None, A16b, A16b, None, None, None) == 1
    del c


def _gemm(lib, codes=A16, xs=A16, bits=8, M=128, K=1024, W=A16b, alpha=A16b, N=256, Y=A16b, ydt=0):
    return lib.hbl_gemm(codes, xs, bits, M, K, W, alpha, N, Y, ydt, None)


def test_gemm_validation(lib):
    assert _gemm(lib, bits=2) == 6
    assert _gemm(lib, ydt=3) == 5
    assert _gemm(lib, K=1000) == 4 and _gemm(lib, N=100) == 4
    assert _gemm(lib, K=64) == 2 and _gemm(lib, K=192) == 4 and _gemm(lib, K=65536) == 2 and _gemm(lib, N=0) == 2 and _gemm(lib, M=-3) == 2
    assert _gemm(lib, M=(1 << 23) + 1) == 2 and _gemm(lib, N=(1 << 20) + 16) == 2
    assert _gemm(lib, codes=None) == 1 and _gemm(lib, alpha=None) == 1 and _gemm(lib, Y=None) == 1
    assert _gemm(lib, Y=MIS) == 4 and _gemm(lib, W=MIS) == 4
    assert _gemm(lib, M=0, codes=None) == 0


def test_quantize_weights_validation(lib):
    q = lib.hbl_quantize_weights
    assert q(A16, 0, 64, 40, 1e-5, A16b, A16b, A16b, 1 << 20, None) == 4          # K % 16
    assert q(A16, 0, 0, 64, 1e-5, A16b, A16b, A16b, 1 << 20, None) == 2           # N = 0
    assert q(A16, 2, 64, 64, 1e-5, A16b, A16b, A16b, 1 << 20, None) == 5          # dtype
    assert q(None, 0, 64, 64, 1e-5, A16b, A16b, A16b, 1 << 20, None) == 1
    assert q(A16, 0, 64, 64, -1.0, A16b, A16b, A16b, 1 << 20, None) == 2          # negative eps
    assert q(MIS, 0, 64, 64, 1e-5, A16b, A16b, A16b, 1 << 20, None) == 4
    assert q(A16, 0, 64, 64, 1e-5, A16b, A16b, A16b, 0, None) == 7                # workspace


def test_forward_validation(lib):
    cfg = hbl.Config(act_bits=8).c()
    f = lib.hbl_forward
    need = hbl.hbl_workspace_bytes(64, 1024, hbl.Config(act_bits=8))
    assert f(A16, 0, 64, 1024, None, A16b, A16b, 256, ctypes.byref(cfg), A16b, 0, A16b, need - 1, None) == 7
    assert f(A16, 0, 64, 1000, None, A16b, A16b, 256, ctypes.byref(cfg), A16b, 0, A16b, need, None) == 3
    assert f(A16, 0, 64, 1024, None, A16b, A16b, 250, ctypes.byref(cfg), A16b, 0, A16b, need, None) == 4
    assert f(A16, 0, 64, 1024, None, None, A16b, 256, ctypes.byref(cfg), A16b, 0, A16b, need, None) == 1
    assert f(A16, 0, 64, 1024, None, A16b, A16b, 256, None, A16b, 0, A16b, need, None) == 1
    assert f(A16, 0, 0, 1024, None, A16b, A16b, 256, ctypes.byref(cfg), A16b, 0, A16b, 0, None) == 0


def test_forward_latent_validation(lib):
    cfg = hbl.Config(act_bits=8).c()
    f = lib.hbl_forward_latent
    M, K, N = 64, 1024, 256
    need = hbl.hbl_workspace_bytes(M, K, hbl.Config(act_bits=8))
    wneed = hbl.hbl_weight_workspace_bytes(N, K)

    def call(X=A16, xdt=0, M=M, K=K, W=A16b, wdt=0, N=N, eps=1e-5, c=ctypes.byref(cfg), Wp=A16b, alpha=A16b,
             Y=A16b, ydt=0, ws=A16b, wsb=need, wws=A16b, wwsb=wneed):
        return f(X, xdt, M, K, None, W, wdt, N, eps, c, Wp, alpha, Y, ydt, ws, wsb, wws, wwsb, None)

    assert call(wdt=4) == 5 and call(xdt=2) == 5 and call(ydt=7) == 5
    assert call(K=1008) == 3                         # a multiple of 16 but not a power of two
    assert call(N=250) == 4                          # N % 16
    assert call(eps=-1.0) == 2
    assert call(W=None) == 1 and call(Wp=None) == 1 and call(alpha=None) == 1 and call(wws=None) == 1
    assert call(X=None) == 1 and call(ws=None) == 1 and call(c=None) == 1
    assert call(W=MIS) == 4 and call(X=MIS) == 4
    assert call(wsb=need - 1) == 7 and call(wwsb=wneed - 1) == 7


def test_quantize_heads_validation(lib):
    q = lib.hbl_quantize_heads
    ok = dict(X=A16, xdt=1, M=8, H=4, D=128, bits=3, eps=1e-5, codes=A16b, scales=A16b)

    def call(**kw):
        a = dict(ok, **kw)
        return q(a["X"], a["xdt"], a["M"], a["H"], a["D"], a["bits"], a["eps"], a["codes"], a["scales"], None)

    assert call(xdt=3) == 5
    assert call(bits=5) == 6 and call(bits=2) == 6
    assert call(D=48) == 2 and call(D=512) == 2 and call(H=0) == 2 and call(M=-1) == 2 and call(eps=-1.0) == 2
    assert call(M=(1 << 40) // 512 + 1, H=4, D=128) == 2
    assert call(X=None) == 1 and call(codes=None) == 1 and call(scales=None) == 1
    assert call(M=0, X=None, codes=None, scales=None) == 0


def test_backward_validation(lib):
    cfg = hbl.Config(act_bits=8).c()
    f = lib.hbl_backward
    M, K, N = 64, 1024, 256
    need = hbl.hbl_backward_workspace_bytes(M, K, N, hbl.Config(act_bits=8), True)
    assert need > hbl.hbl_backward_workspace_bytes(M, K, N, hbl.Config(act_bits=8), False)

    def call(dY=A16, dydt=0, X=A16b, xdt=0, M=M, K=K, W=A16, alpha=A16b, N=N, c=ctypes.byref(cfg), dX=A16,
             dW=A16b, ws=A16, wsb=need):
        return f(dY, dydt, X, xdt, M, K, None, W, alpha, N, c, dX, dW, ws, wsb, None)

    assert call(dydt=3) == 5 and call(xdt=3) == 5
    assert call(K=256) == 2                       # below 512
    assert call(K=1008) == 3                      # not a power of two
    assert call(N=250) == 4
    assert call(dX=None) == 1 and call(W=None) == 1 and call(ws=None) == 1
    assert call(wsb=need - 1) == 7
    assert call(M=0, dY=None, X=None, dX=None, ws=None) == 0
    with pytest.raises(hbl.HblError):
        hbl.hbl_backward_workspace_bytes(M, K, (1 << 21) + 16, hbl.Config(act_bits=8))


def test_base3_size_and_pack_validation(lib):
    assert hbl.hbl_base3_weight_bytes(4096, 8192) == 4096 * 16 * 103       # ceil(8192 / 80) = 103 vectors
    assert hbl.hbl_base3_weight_bytes(3, 80) == 3 * 16 and hbl.hbl_base3_weight_bytes(3, 96) == 3 * 32
    with pytest.raises(hbl.HblError):
        hbl.hbl_base3_weight_bytes(16, 40)                                   # K % 16
    p = lib.hbl_pack_base3
    assert p(A16, 64, 40, A16b, None) == 4 and p(A16, 0, 64, A16b, None) == 2
    assert p(None, 64, 64, A16b, None) == 1 and p(A16, 64, 64, None, None) == 1
    assert p(MIS, 64, 64, A16b, None) == 4 and p(A16, 64, 64, MIS, None) == 4


def test_base3_gemm_and_forward_validation(lib):
    g = lib.hbl_gemm_base3

    def gemm(codes=A16, xs=A16b, bits=8, M=1, K=8192, W=A16, alpha=A16b, N=4096, Y=A16b, ydt=0):
        return g(codes, xs, bits, M, K, W, alpha, N, Y, ydt, None)

    assert gemm(bits=2) == 6 and gemm(ydt=3) == 5
    assert gemm(M=5) == 2 and gemm(M=-1) == 2 and gemm(K=16384 + 16) == 2 and gemm(K=8) == 2
    assert gemm(K=1000) == 4 and gemm(N=0) == 2 and gemm(N=(1 << 20) + 1) == 2
    assert gemm(codes=None) == 1 and gemm(W=None) == 1 and gemm(Y=None) == 1
    assert gemm(W=MIS) == 4 and gemm(Y=MIS) == 4
    assert gemm(M=0, codes=None) == 0
    cfg = hbl.Config(act_bits=4).c()
    f = lib.hbl_forward_base3
    need = hbl.hbl_workspace_bytes(4, 8192, hbl.Config(act_bits=4))

    def fwd(X=A16, M=4, K=8192, W=A16b, N=4096, c=ctypes.byref(cfg), wsb=need):
        return f(X, 0, M, K, None, W, A16b, N, c, A16b, 0, A16, wsb, None)

    assert fwd(wsb=need - 1) == 7 and fwd(M=5) == 2 and fwd(K=32768) == 2 and fwd(K=8000) == 3
    assert fwd(X=None) == 1 and fwd(W=None) == 1 and fwd(c=None) == 1
    assert fwd(M=0, X=None, W=None) == 0


def test_binding_checks_buffer_sizes():
    """The binding checks every caller-provided buffer against the size its
    shape needs (the C ABI cannot: it takes bare pointers)."""
    import torch
    hbl._fits(torch.empty(16, dtype=torch.uint8), 16, "x")
    hbl._fits(None, 1 << 40, "x")
    with pytest.raises(ValueError):
        hbl._fits(torch.empty(15, dtype=torch.uint8), 16, "x")
    with pytest.raises(ValueError):
        hbl._fits(torch.empty(3, dtype=torch.float32), 16, "x")


def _peaks_lib():
    import ctypes
    from bit_bitlinear_amd import build as hbl_build
    lib = ctypes.CDLL(hbl_build.PEAKS_LIB)
    lib.hbl_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hbl_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_void_p]
    lib.hbl_peak_mfma_ops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
    lib.hbl_peak_mfma_ops.restype = ctypes.c_int64
    lib.hbl_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.hbl_peak_read_sink_len.argtypes = [ctypes.c_int64]
    lib.hbl_peak_read_sink_len.restype = ctypes.c_int64
    lib.hbl_peak_empty.argtypes = [ctypes.c_int32, ctypes.c_void_p]
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.hbl_peak_lds.argtypes = [I32, P, I64, I32, I32, P, I64, P, I64, P]
    return lib


def test_peaks_library_exports_and_host_checks():
    """The probe library the benchmark uses for measured ceilings: every
    symbol include/hbl_peaks.h declares is exported, the op counts are the
    instructions' dense work, and bad arguments are refused before any launch."""
    import os
    lib = _peaks_lib()
    names = hbl.declared_symbols(os.path.join(os.path.dirname(hbl.HEADER_PATH), "hbl_peaks.h"))
    assert names == ["hbl_peak_copy", "hbl_peak_empty", "hbl_peak_lds", "hbl_peak_mfma", "hbl_peak_mfma_ops",
                     "hbl_peak_read", "hbl_peak_read_sink_len", "hbl_peak_write"]
    assert all(hasattr(lib, n) for n in names)
    # 4 waves x 4 instructions per round: i8 32x32x32, FP6 x FP4 32x32x64, bf16 32x32x16
    assert lib.hbl_peak_mfma_ops(0, 1, 1) == 16 * 2 * 32 * 32 * 32
    assert lib.hbl_peak_mfma_ops(1, 3, 5) == 16 * 2 * 32 * 32 * 64 * 15
    assert lib.hbl_peak_mfma_ops(2, 2048, 2000) == 16 * 2 * 32 * 32 * 16 * 2048 * 2000
    for bad in ((3, 1, 1), (0, 0, 1), (0, 1, 0), (0, (1 << 20) + 1, 1), (0, 1, (1 << 24) + 1)):
        assert lib.hbl_peak_mfma_ops(*bad) == -1
    assert lib.hbl_peak_mfma(3, 16, 256, 1, 1, None) == 1            # unknown kind
    assert lib.hbl_peak_mfma(0, 16, 255, 1, 1, None) == 1            # out too short
    assert lib.hbl_peak_mfma(0, None, 256, 1, 1, None) == 1          # no output
    assert lib.hbl_peak_copy(16, 4096, 17, None) == 1                # not a multiple of 16
    assert lib.hbl_peak_copy(16, 32, 64, None) == 1                  # overlapping
    assert lib.hbl_peak_copy(None, 4096, 16, None) == 1              # null
    assert lib.hbl_peak_copy(24, 4096, 16, None) == 1                # misaligned
    assert lib.hbl_peak_copy(16, 4096, 0, None) == 0                 # nothing to do
    assert lib.hbl_peak_read_sink_len(8 << 20) == (8 << 20) // 16 // 1024 * 256
    assert lib.hbl_peak_read_sink_len(17) == -1
    assert lib.hbl_peak_read(16, 4096, 32, 255, None) == 1           # sink too short (one block of 256)
    assert lib.hbl_peak_read(24, 4096, 32, 256, None) == 1           # misaligned
    assert lib.hbl_peak_read(16, 0, 32, 256, None) == 1              # nothing to read
    assert lib.hbl_peak_empty(0, None) == 1 and lib.hbl_peak_empty((1 << 20) + 1, None) == 1
    # data-path probe: kind, source size (a power of two in [64 KiB, 1 GiB]), counts and buffer lengths
    good = (1, 4096, 1 << 21, 4, 10, 64, 8, 128, 4, None)
    def lds(**kw):
        a = list(good)
        for k, v in kw.items():
            a[["kind", "src", "bytes", "blocks", "iters", "clk", "clk_len", "sink", "sink_len", "s"].index(k)] = v
        return lib.hbl_peak_lds(*a)
    assert lds(kind=5) == 1 and lds(kind=-1) == 1
    assert lds(bytes=(1 << 21) + 16) == 1 and lds(bytes=1 << 15) == 1 and lds(bytes=1 << 31) == 1
    assert lds(src=None) == 1 and lds(src=4104) == 1
    assert lds(blocks=0) == 1 and lds(blocks=(1 << 20) + 1) == 1
    assert lds(iters=1) == 1 and lds(iters=(1 << 24) + 1) == 1
    assert lds(clk_len=7) == 1 and lds(clk=None) == 1
    assert lds(sink_len=3) == 1 and lds(sink=None) == 1
    lib.hbl_peak_write.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    assert lib.hbl_peak_write(4096, 17, None) == 1                  # not a multiple of 16
    assert lib.hbl_peak_write(None, 16, None) == 1                  # null
    assert lib.hbl_peak_write(4104, 16, None) == 1                  # misaligned
    assert lib.hbl_peak_write(4096, 0, None) == 0                   # nothing to do


def test_fp4_fp6_validation(lib):
    """The FP4-weight INT4 path: size queries, weight conversion, FP6 codes,
    the FP6 x FP4 GEMM and the forward reject bad arguments on the host."""
    c4, c8 = hbl.Config(act_bits=4), hbl.Config(act_bits=8)
    assert hbl.hbl_fp4_weight_bytes(4096, 16384) == 4096 * 8192
    assert hbl.hbl_fp6_codes_bytes(8192, 16384) == 8192 * 12288
    assert hbl.hbl_forward_fp4_workspace_bytes(8192, 16384, c4) >= 8192 * 12288 + 8192 * 4
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_forward_fp4_workspace_bytes(8192, 16384, c8)           # INT8 codes have no FP6 form
    assert e.value.status == 6
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_forward_fp4_workspace_bytes(8, 256, c4)                # K < 512
    assert e.value.status == 2
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_fp6_codes_bytes(8, 576)                                # K % 128
    assert e.value.status == 4
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_fp4_weight_bytes(16, 64)                               # the FP4 format holds whole K steps of 128
    assert e.value.status == 4
    assert lib.hbl_pack_fp4(None, 16, 128, A16b, None) == 1
    assert lib.hbl_pack_fp4(A16, 16, 40, A16b, None) == 4
    assert lib.hbl_pack_fp4(A16, 16, 64, A16b, None) == 4              # K % 128
    assert lib.hbl_pack_fp4(MIS, 16, 128, A16b, None) == 4
    cc4, cc8 = c4.c(), c8.c()
    q6 = lib.hbl_quantize_activations_fp6
    assert q6(A16, 0, 8, 1024, None, ctypes.byref(cc8), A16b, A16b, None) == 6
    assert q6(A16, 0, 8, 256, None, ctypes.byref(cc4), A16b, A16b, None) == 2
    assert q6(A16, 0, 8, 1536, None, ctypes.byref(cc4), A16b, A16b, None) == 3
    assert q6(A16, 3, 8, 1024, None, ctypes.byref(cc4), A16b, A16b, None) == 5
    assert q6(None, 0, 8, 1024, None, ctypes.byref(cc4), A16b, A16b, None) == 1
    assert q6(A16, 0, 0, 1024, None, ctypes.byref(cc4), None, None, None) == 0   # M = 0 queues nothing
    g = lib.hbl_gemm_fp6fp4
    assert g(A16, A16b, 8, 384, A16b, A16b, 64, A16b, 0, None) == 2              # K < 512
    assert g(A16, A16b, 8, 576, A16b, A16b, 64, A16b, 0, None) == 4              # K % 128
    assert g(A16, A16b, 8, 1024, A16b, A16b, 40, A16b, 0, None) == 4             # N % 16
    assert g(A16, A16b, 8, 1024, A16b, A16b, 64, A16b, 9, None) == 5
    assert g(A16, A16b, 8, 1024, MIS, A16b, 64, A16b, 0, None) == 4
    assert g(None, A16b, 8, 1024, A16b, A16b, 64, A16b, 0, None) == 1
    f = lib.hbl_forward_fp4
    assert f(A16, 0, 8, 1024, None, A16b, A16b, 64, ctypes.byref(cc4), A16b, 0, A16b, 16, None) == 7
    assert f(A16, 0, 8, 1024, None, A16b, A16b, 64, ctypes.byref(cc8), A16b, 0, A16b, 1 << 20, None) == 6
    assert f(A16, 0, 8, 1024, None, None, A16b, 64, ctypes.byref(cc4), A16b, 0, A16b, 1 << 20, None) == 1
    assert f(A16, 0, 8, 1024, None, A16b, A16b, 72, ctypes.byref(cc4), A16b, 0, A16b, 1 << 20, None) == 4


def test_forward_noalloc_host_checks(lib):
    """The no-allocation forward rejects on the host, before any HIP call:
    shapes whose workspace exceeds the static scratch, and bad arguments."""
    c8 = hbl.Config(act_bits=8).c()
    f = lib.hbl_forward_noalloc
    # 8192 x 8192 INT8 codes need 64 MiB > HBL_NOALLOC_SCRATCH_BYTES
    assert f(A16, 0, 8192, 8192, None, A16b, A16b, 256, ctypes.byref(c8), A16b, 0, None) == 7
    assert f(A16, 0, 8, 300, None, A16b, A16b, 256, ctypes.byref(c8), A16b, 0, None) == 3   # K not a power of two
    assert f(None, 0, 8, 256, None, A16b, A16b, 256, ctypes.byref(c8), A16b, 0, None) == 1
    assert f(MIS, 0, 8, 256, None, A16b, A16b, 256, ctypes.byref(c8), A16b, 0, None) == 4
    assert f(None, 0, 0, 256, None, None, None, 256, ctypes.byref(c8), None, 0, None) == 0   # M = 0: nothing
    bad = hbl.Config(act_bits=5).c()
    assert f(A16, 0, 8, 256, None, A16b, A16b, 256, ctypes.byref(bad), A16b, 0, None) == 6
    assert hbl.HBL_NOALLOC_SCRATCH_BYTES == 32 << 20
