"""hbl_forward_noalloc through the C ABI: the forward with its workspace in
the library's static device array must give hbl_forward's result bit for bit,
on two calls in a row, the second with a smaller input (the array keeps the
first call's contents), and must reject a shape whose workspace exceeds the
array.  It must pass alone in a fresh process and after the other tests."""
import numpy as np
import pytest

import bit_bitlinear_amd as hbl
import workloads
from parity import to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(M, K, N, bits, had, xdt, ydt, seed):
    import torch
    rng = np.random.default_rng(seed)
    X, _ = workloads.x_outlier_gaussian(rng, M, K, 4, 30.0)
    W = workloads.w_latent(rng, N, K)
    Xd = to_dev(workloads.f32_to_bf16_bits(X) if xdt == "bf16" else X)
    cfg = hbl.Config(act_bits=bits, hadamard=had)
    Wp, alpha = hbl.hbl_quantize_weights(to_dev(W))
    yt = torch.float32 if ydt == "f32" else torch.bfloat16
    return Xd, Wp, alpha, cfg, yt


@pytest.mark.parametrize("first,second", [
    ((4096, 2048, 2048, 8, True, "bf16", "bf16"), (300, 1024, 512, 4, True, "f32", "f32")),
    ((1024, 4096, 4096, 4, False, "bf16", "bf16"), (16, 8192, 1024, 4, True, "f32", "bf16")),
])
def test_forward_noalloc_matches_forward_twice(first, second):
    import torch
    print("[case] noalloc %s then %s" % (first, second), flush=True)
    for i, (M, K, N, bits, had, xdt, ydt) in enumerate((first, second)):
        Xd, Wp, alpha, cfg, yt = _case(M, K, N, bits, had, xdt, ydt, seed=M + K + N + i)
        assert hbl.hbl_workspace_bytes(M, K, cfg) <= hbl.HBL_NOALLOC_SCRATCH_BYTES
        Y_ref = hbl.hbl_forward(Xd, Wp, alpha, N, cfg, y_dtype=yt)
        Y = hbl.hbl_forward_noalloc(Xd, Wp, alpha, N, cfg, y_dtype=yt)
        Y2 = torch.empty_like(Y)
        hbl.hbl_forward_noalloc(Xd, Wp, alpha, N, cfg, Y=Y2)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(Y), to_host(Y_ref)), "call %d differs from hbl_forward" % i
        assert np.array_equal(to_host(Y2), to_host(Y_ref)), "repeat of call %d differs" % i


def test_forward_noalloc_rejects_oversized_shape():
    import torch
    cfg = hbl.Config(act_bits=8)
    M, K, N = 8192, 8192, 64
    assert hbl.hbl_workspace_bytes(M, K, cfg) > hbl.HBL_NOALLOC_SCRATCH_BYTES
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda:0")
    Wp = torch.zeros((N, K // 4), dtype=torch.uint8, device="cuda:0")
    alpha = torch.ones(1, dtype=torch.float32, device="cuda:0")
    with pytest.raises(hbl.HblError) as e:
        hbl.hbl_forward_noalloc(X, Wp, alpha, N, cfg)
    assert e.value.status == 7
