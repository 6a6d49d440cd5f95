"""The probe kernels behind the benchmark's measured ceilings (libhbl_peaks.so)
run and do what include/hbl_peaks.h says: the copy copies, the write writes
its pattern, the data-path probe records its clocks for every kind."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _lib():
    from bit_bitlinear_amd import build as hbl_build
    lib = ctypes.CDLL(hbl_build.PEAKS_LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.hbl_peak_copy.argtypes = [P, P, I64, P]
    lib.hbl_peak_write.argtypes = [P, I64, P]
    lib.hbl_peak_read.argtypes = [P, I64, P, I64, P]
    lib.hbl_peak_read_sink_len.argtypes = [I64]
    lib.hbl_peak_read_sink_len.restype = I64
    lib.hbl_peak_lds.argtypes = [I32, P, I64, I32, I32, P, I64, P, I64, P]
    lib.hbl_peak_mfma.argtypes = [I32, P, I64, I32, I32, P]
    return lib


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def test_copy_and_write_probes():
    import torch
    print("[case] peak copy / write", flush=True)
    lib = _lib()
    n = (1 << 20) + 48  # bytes: a ragged last block
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    assert lib.hbl_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, _stream()) == 0
    out = torch.zeros(n // 4, dtype=torch.int32, device="cuda:0")
    assert lib.hbl_peak_write(ctypes.c_void_p(out.data_ptr()), n, _stream()) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    # vector i of block b = i // 1024, thread t = i % 256 holds (b * 1024 + t, b, 0x5A5A5A5A, 0)
    got = out.cpu().numpy().view(np.uint32).reshape(-1, 4)
    i = np.arange(got.shape[0], dtype=np.int64)
    b, t = i // 1024, i % 256
    want = np.stack([(b * 1024 + t).astype(np.uint32), b.astype(np.uint32),
                     np.full_like(b, 0x5A5A5A5A, dtype=np.uint32), np.zeros_like(b, dtype=np.uint32)], 1)
    assert np.array_equal(got, want)


def test_read_and_mfma_probes_run():
    import torch
    print("[case] peak read / mfma", flush=True)
    lib = _lib()
    size = 1 << 20
    src = torch.ones(size // 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(lib.hbl_peak_read_sink_len(size), dtype=torch.int32, device="cuda:0")
    assert lib.hbl_peak_read(ctypes.c_void_p(src.data_ptr()), size, ctypes.c_void_p(sink.data_ptr()), sink.numel(),
                             _stream()) == 0
    out = torch.zeros(8 * 256, dtype=torch.int32, device="cuda:0")
    for kind in range(3):
        assert lib.hbl_peak_mfma(kind, ctypes.c_void_p(out.data_ptr()), out.numel(), 8, 4, _stream()) == 0
    torch.cuda.synchronize()
    assert not sink.any()  # all-ones data never folds to the sink's value


@pytest.mark.parametrize("kind", [0, 1, 2, 3, 4])
def test_lds_probe_records_its_clock(kind):
    import torch
    print("[case] peak lds kind %d" % kind, flush=True)
    lib = _lib()
    blocks = 16
    src = torch.ones((2 << 20) // 4, dtype=torch.int32, device="cuda:0")
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda:0")
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda:0")
    assert lib.hbl_peak_lds(kind, ctypes.c_void_p(src.data_ptr()), src.numel() * 4, blocks, 64,
                            ctypes.c_void_p(clk.data_ptr()), clk.numel(), ctypes.c_void_p(sink.data_ptr()),
                            sink.numel(), _stream()) == 0
    torch.cuda.synchronize()
    c = clk.view(blocks, 2).cpu().numpy().astype(np.float64)
    assert (c > 0).all()
    ghz = c[:, 0] / (c[:, 1] / 100e6) / 1e9  # shader cycles over 100 MHz real-time ticks
    assert ((ghz > 0.3) & (ghz < 4.0)).all(), ghz
